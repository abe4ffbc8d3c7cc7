"""The multi-threaded host-CPU scoring pass (libnf4cpu.so) against the oracle.

Runs without a GPU.  Codes, block absmax, int8 absmax and scales bit-exact;
errors within 1e-9 relative (both sum exact squares in fp64, in different
orders); bitwise the same for 1 and 8 threads.  Inputs: ragged sizes, zero
blocks and groups, negative zeros, subnormal and tiny-normal absmax, values
up to 3.4e38, outliers; bf16 and fp16; double quantisation on and off.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import quantized_lora_fine_nf4_amd as q
import synth
from quantized_lora_fine_nf4_amd import cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _layers(dtype):
    rng = np.random.default_rng(31 + dtype)
    L = [synth.generate_raw(800 + k, n, dtype=dtype, outlier_frac=0.002)
         for k, n in enumerate([1, 2, 63, 64, 65, 1000, 16383, 16384, 16385, 2 * 16384 + 77,
                                100_003])]
    z = np.zeros(2 * 16384 + 100, np.uint16)
    z[rng.integers(0, z.size, 50)] = 0x8000
    L.append(z)
    m = synth.generate_raw(850, 3 * 16384 + 640, dtype=dtype)
    m[16384:2 * 16384] = 0
    for b in rng.integers(0, m.size // 64, 30):
        m[64 * b: 64 * b + 64] = 0
    L.append(m)
    sub = rng.integers(1, 0x80 if dtype == q.NF4_BF16 else 0x400, 64 * 200).astype(np.uint16)
    sub |= (rng.integers(0, 2, sub.size).astype(np.uint16) << 15)
    L.append(sub)
    if dtype == q.NF4_BF16:
        e = rng.integers(0x0A00, 0x0D00, 64 * 200).astype(np.uint16)
        e |= (rng.integers(0, 2, e.size).astype(np.uint16) << 15)
        L.append(e)
        h = rng.integers(0x7E00, 0x7F7F, 64 * 40).astype(np.uint16)
        h |= (rng.integers(0, 2, h.size).astype(np.uint16) << 15)
        L.append(h)
    return L


@pytest.mark.parametrize("dq", [False, True], ids=["nodq", "dq"])
@pytest.mark.parametrize("dtype", [q.NF4_BF16, q.NF4_FP16], ids=["bf16", "fp16"])
def test_cpu_pass_matches_oracle(dtype, dq):
    f = q.fmt(dtype, dq)
    ws = _layers(dtype)
    got = cpu.layer_error(ws, f, threads=4)
    for i, w in enumerate(ws):
        ref = oracle.layer_error(w, dtype, dq)
        assert np.array_equal(got["codes"][i], ref["codes"]), i
        assert np.array_equal(got["absmax"][i].view(np.uint32), ref["absmax"].view(np.uint32)), i
        if dq:
            assert np.array_equal(got["qabsmax"][i], ref["qabsmax"]), i
            assert np.array_equal(got["scale2"][i].view(np.uint32), ref["scale2"].view(np.uint32)), i
        e, r = got["err"][i], ref["err"]
        assert (e == r == 0.0) or abs(e - r) <= 1e-9 * r, (i, e, r)


def test_cpu_pass_is_deterministic_across_thread_counts():
    f = q.fmt(q.NF4_BF16, True)
    ws = [synth.generate_raw(900 + k, n) for k, n in enumerate([70_001, 16384 * 9, 5, 333_333])]
    a = cpu.layer_error(ws, f, threads=1)
    b = cpu.layer_error(ws, f, threads=8)
    assert np.array_equal(a["err"].view(np.int64), b["err"].view(np.int64))
    for k in ("codes", "qabsmax", "scale2"):
        for x, y in zip(a[k], b[k]):
            assert np.array_equal(x, y)


def test_cpu_pass_toy_stack_selection_equals_oracle():
    from synth import configs
    cfg = configs.BY_NAME["toy"]
    f = q.fmt(cfg.dtype, cfg.dq)
    ws = [synth.generate(cfg, i) for i in range(cfg.n_layers)]
    got = cpu.layer_error(ws, f)
    ref = np.array([oracle.layer_error(w, cfg.dtype, cfg.dq)["err"] for w in ws])
    assert np.all(np.abs(got["err"] - ref) <= 1e-9 * ref)
    cost = [oracle.promote_cost(w.size, cfg.dq) for w in ws]
    assert np.array_equal(oracle.select_topk(got["err"], cost, -1, cfg.kcap)[0],
                          oracle.select_topk(ref, cost, -1, cfg.kcap)[0])


def test_cpu_pass_arguments():
    L = cpu.lib()
    f = q.fmt()
    w = np.zeros(128, np.uint16)
    c = np.zeros(64, np.uint8)
    qa = np.zeros(2, np.int8)
    s2 = np.zeros(1, np.float32)
    err = np.zeros(1, np.float64)
    good = q.nf4_layer(128, w.ctypes.data, c.ctypes.data, None, qa.ctypes.data, s2.ctypes.data,
                       None)

    def call(layer=good, nl=1, fmt=f, e=err.ctypes.data):
        arr = (q.nf4_layer * 1)(layer)
        return L.nf4_cpu_layer_error(arr, nl, fmt, e, 1)
    assert call() == q.NF4_OK
    assert call(nl=0) == q.NF4_E_ARG
    assert call(e=None) == q.NF4_E_ARG
    assert call(fmt=q.nf4_format(0, 32, 256)) == q.NF4_E_UNSUPPORTED
    assert call(fmt=q.nf4_format(5, 64, 256)) == q.NF4_E_UNSUPPORTED
    for fld in ("w", "codes", "qabsmax", "scale2"):
        bad = q.nf4_layer(128, good.w, good.codes, None, good.qabsmax, good.scale2, None)
        setattr(bad, fld, None)
        assert call(layer=bad) == q.NF4_E_ARG, fld
    nodq = q.nf4_layer(128, good.w, good.codes, None, None, None, None)
    assert call(layer=nodq, fmt=q.fmt(dq=False)) == q.NF4_E_ARG      # absmax required
    assert cpu.max_threads() >= 1


def test_cpu_library_exports_its_header():
    text = open(os.path.join(ROOT, "include", "nf4_cpu.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(nf4_cpu_[a-z_]+)\s*\(", text))
    assert names == {"nf4_cpu_layer_error", "nf4_cpu_max_threads"}
    L = ctypes.CDLL(cpu.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_cpu_pass_isa_paths_agree_bitwise():
    """The AVX-512 and AVX2 tile paths give the same bits (each run in its own
    process, the path chosen with NF4_CPU_ISA)."""
    import subprocess
    import sys
    code = (
        "import sys, numpy as np; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "import quantized_lora_fine_nf4_amd as q, synth\n"
        "from quantized_lora_fine_nf4_amd import cpu\n"
        "ws = [synth.generate_raw(950 + k, n, dtype=d) for k, (n, d) in enumerate("
        "[(70_001, 0), (16384 * 3 + 5, 1), (333, 0)])]\n"
        "outs = []\n"
        "for dt in (0, 1):\n"
        "    o = cpu.layer_error([w for w in ws], q.fmt(dt, True), threads=4)\n"
        "    outs.append(np.concatenate([o['err'].view(np.uint8)] + o['codes'] + "
        "[x.view(np.uint8) for x in o['qabsmax'] + o['scale2']]))\n"
        "sys.stdout.write(np.concatenate(outs).tobytes().hex())\n"
    ) % (ROOT, os.path.join(ROOT, "tests"))
    res = {}
    for isa in ("avx2", "auto"):
        env = dict(os.environ, NF4_CPU_ISA=isa)
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        res[isa] = r.stdout
    assert res["avx2"] == res["auto"] and len(res["avx2"]) > 1000
