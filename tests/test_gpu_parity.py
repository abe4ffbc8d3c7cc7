"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact on codes, absmax, int8 absmax, second-level scales, dequantised
16-bit values, the selected set and K; per-layer errors within 1e-5 relative
(the design aims far below: fp32 inside a 64-block, fp64 beyond).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import quantized_lora_fine_nf4_amd as q
import synth
from conftest import print_case
from gpu_util import POISON, compare_layer, layer_error, layerset, np_of, poison, rel_err, workspace
from synth import configs

pytestmark = pytest.mark.gpu

ERR_RTOL = 1e-5
DTYPES = {"bf16": q.NF4_BF16, "fp16": q.NF4_FP16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    q.lib()  # fails loudly if the HIP library is missing
    yield
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
def _edge_layers(dtype):
    """Ragged sizes and special contents, one grouped call."""
    rng = np.random.default_rng(1234 + dtype)
    L = []
    for k, n in enumerate([1, 2, 3, 63, 64, 65, 127, 129, 1000, 16383, 16384, 16385,
                           2 * 16384 + 77, 100_003]):
        L.append((f"n{n}", synth.generate_raw(500 + k, n, dtype=dtype, outlier_frac=0.002)))
    z = np.zeros(2 * 16384 + 100, np.uint16)
    z[rng.integers(0, z.size, 50)] = 0x8000                      # negative zeros
    L.append(("zeros", z))
    m = synth.generate_raw(600, 5 * 16384 + 640, dtype=dtype)
    m[16384:2 * 16384] = 0                                        # a whole zero group
    for b in rng.integers(0, m.size // 64, 40):
        m[64 * b: 64 * b + 64] = 0                                # zero blocks
    L.append(("zero_blocks", m))
    sub = rng.integers(1, 0x80 if dtype == q.NF4_BF16 else 0x400, 64 * 300).astype(np.uint16)
    sub |= (rng.integers(0, 2, sub.size).astype(np.uint16) << 15)
    L.append(("subnormal_absmax", sub))
    if dtype == q.NF4_BF16:
        # normal fp32 absmax below 2^-100 (the kernels' prescale path)
        e = rng.integers(0x0A00, 0x0D00, 64 * 300).astype(np.uint16)   # ~2^-108 .. 2^-102
        e |= (rng.integers(0, 2, e.size).astype(np.uint16) << 15)
        L.append(("tiny_normal_absmax", e))
    one = synth.generate_raw(700, 64 * 256 * 2, dtype=dtype)
    x = oracle.from16(one, dtype)
    x[777] *= 200.0
    one = oracle.to16_rne(x, dtype)
    L.append(("single_outlier", one))
    return L


@pytest.mark.parametrize("dq", [False, True], ids=["nodq", "dq"])
@pytest.mark.parametrize("dtname", ["bf16", "fp16"])
def test_edge_layers_fused_pass_and_dequant(dtname, dq):
    dtype = DTYPES[dtname]
    f = q.fmt(dtype, dq)
    layers = _edge_layers(dtype)
    print_case("edge layers", dtname, "dq" if dq else "nodq", [nm for nm, _ in layers])
    ls = layerset([w for _, w in layers], f)
    err = layer_error(ls, f)
    torch.cuda.synchronize()
    errs = err.cpu().numpy()
    ws = workspace(ls.ns, f)
    q.nf4_dequantize(ls, f, ws)
    torch.cuda.synchronize()
    worst = 0.0
    for i, (nm, w) in enumerate(layers):
        ref = compare_layer(ls, i, w, dtype, dq, check_out=True)
        r = rel_err(errs[i], ref["err"])
        worst = max(worst, r)
        assert r <= ERR_RTOL, (nm, errs[i], ref["err"])
        if ref["err"] == 0.0:
            assert errs[i] == 0.0, nm
    print(f"[edge {dtname} dq={dq}] worst relative error gap {worst:.3e}", flush=True)


@pytest.mark.parametrize("dq", [False, True], ids=["nodq", "dq"])
@pytest.mark.parametrize("dtname", ["bf16", "fp16"])
def test_quantize_then_dequantize_matches_oracle(dtname, dq):
    """nf4_quantize (separate kernel instance, no error) + nf4_dequantize."""
    dtype = DTYPES[dtname]
    f = q.fmt(dtype, dq)
    layers = _edge_layers(dtype)
    if dtype == q.NF4_BF16:
        big = np.array([0x7F00, 0xFE7F, 0x7E12, 0x0001] * 16 * 40, np.uint16)   # up to 1.7e38
        layers.append(("huge", big))
    print_case("quantize+dequantize", dtname, dq)
    ls = layerset([w for _, w in layers], f)
    ws = workspace(ls.ns, f)
    q.nf4_quantize(ls, f, ws)
    q.nf4_dequantize(ls, f, ws)
    torch.cuda.synchronize()
    for i, (nm, w) in enumerate(layers):
        compare_layer(ls, i, w, dtype, dq, check_out=True)


def test_standalone_double_quant_equals_fused():
    f = q.fmt(q.NF4_BF16, True)
    layers = _edge_layers(q.NF4_BF16)
    ls = layerset([w for _, w in layers], f)
    ws = workspace(ls.ns, f)
    print_case("double quant standalone")
    q.nf4_quantize(ls, f, ws)
    torch.cuda.synchronize()
    q_fused = ls.qabsmax.clone()
    s_fused = ls.scale2.clone()
    ls.qabsmax.fill_(77)
    ls.scale2.fill_(-1.0)
    q.nf4_double_quant(ls, f, ws)
    torch.cuda.synchronize()
    for i, (nm, w) in enumerate(layers):
        nb = (w.size + 63) // 64
        ng = (nb + 255) // 256
        a, b = ls.a_off[i], ls.s_off[i]
        assert torch.equal(ls.qabsmax[a:a + nb], q_fused[a:a + nb]), nm
        assert torch.equal(ls.scale2[b:b + ng].view(torch.int32), s_fused[b:b + ng].view(torch.int32)), nm
        ref_q, ref_s = oracle.double_quant(np_of(ls.absmax_of(i), np.float32))
        assert np.array_equal(np_of(ls.qabsmax_of(i), np.int8), ref_q)


def test_fused_absmax_optional_with_double_quant():
    f = q.fmt(q.NF4_BF16, True)
    w = synth.generate_raw(9, 16384 * 3 + 5)
    ls = layerset([w], f, with_absmax=False)
    err = layer_error(ls, f)
    torch.cuda.synchronize()
    ref = compare_layer(ls, 0, w, q.NF4_BF16, True)
    assert rel_err(err.item(), ref["err"]) <= ERR_RTOL


# --------------------------------------------------------------------------
def _all_bf16_below(a_bits: int, dtype) -> np.ndarray:
    """Every non-negative 16-bit pattern up to a_bits, both signs."""
    pos = np.arange(0, a_bits + 1, dtype=np.uint32).astype(np.uint16)
    return np.concatenate([pos, pos | np.uint16(0x8000)])


def _blocks_with_absmax(a_bits: int, vals: np.ndarray) -> np.ndarray:
    per = 63
    nblk = (vals.size + per - 1) // per
    padded = np.resize(vals, nblk * per).reshape(nblk, per)
    out = np.empty((nblk, 64), np.uint16)
    out[:, 0] = a_bits
    out[:, 1:] = padded
    return out.ravel()


@pytest.mark.parametrize("dtname", ["bf16", "fp16"])
def test_encode_every_16bit_value_for_sampled_absmax(dtname):
    """For each sampled absmax a: every 16-bit x with |x| <= a, encoded by both
    kernel instances (quantize, fused error) and compared with the oracle."""
    dtype = DTYPES[dtname]
    rng = np.random.default_rng(99 + dtype)
    if dtype == q.NF4_BF16:
        a_list = list(rng.integers(0x3000, 0x4400, 150)) + [0x3F80, 0x0080, 0x0005, 0x007F,
                                                             0x0C00, 0x0D80, 0x7F7F, 0x5F00]
    else:
        a_list = list(rng.integers(0x1000, 0x7800, 40)) + [0x3C00, 0x0001, 0x03FF, 0x0400, 0x7BFF]
    ws_list = [_blocks_with_absmax(int(a), _all_bf16_below(int(a), dtype)) for a in a_list]
    for dq in (False, True):
        f = q.fmt(dtype, dq)
        print_case("exhaustive encode", dtname, "dq" if dq else "nodq", len(ws_list), "absmax values")
        ls = layerset(ws_list, f, with_out=False)
        q.nf4_quantize(ls, f, workspace(ls.ns, f))
        torch.cuda.synchronize()
        codes_q = [np_of(ls.codes_of(i), np.uint8).copy() for i in range(len(ws_list))]
        poison(ls)
        err = layer_error(ls, f)
        torch.cuda.synchronize()
        errs = err.cpu().numpy()
        for i, w in enumerate(ws_list):
            ref = compare_layer(ls, i, w, dtype, dq)
            assert np.array_equal(codes_q[i], ref["codes"])
            assert rel_err(errs[i], ref["err"]) <= ERR_RTOL


# --------------------------------------------------------------------------
def test_toy_stack_end_to_end():
    """Toy 2-block fp16 decoder: fused pass, top-K=2, dequant of the rest."""
    cfg = configs.TOY
    f = q.fmt(cfg.dtype, cfg.dq)
    ws_list = [synth.generate(cfg, i) for i in range(cfg.n_layers)]
    print_case("toy stack")
    ls = layerset(ws_list, f)
    err = layer_error(ls, f)
    cost = torch.tensor([q.aqlora_promote_cost(n, f) for n in ls.ns], dtype=torch.int64,
                        device="cuda")
    sel = torch.full((cfg.n_layers,), 9, dtype=torch.uint8, device="cuda")
    kout = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    sws = torch.empty(q.aqlora_workspace_bytes(cfg.n_layers), dtype=torch.uint8, device="cuda")
    q.aqlora_select_topk(err, cost, -1, cfg.kcap, sel, kout, sws)
    keep = None
    torch.cuda.synchronize()
    errs = err.cpu().numpy()
    refs = []
    for i in range(cfg.n_layers):
        ref = compare_layer(ls, i, ws_list[i], cfg.dtype, cfg.dq)
        assert rel_err(errs[i], ref["err"]) <= ERR_RTOL
        refs.append(ref)
    ref_err = np.array([r["err"] for r in refs])
    ref_cost = np.array([oracle.promote_cost(n, cfg.dq) for n in cfg.sizes])
    ref_sel, ref_k = oracle.select_topk(ref_err, ref_cost, -1, cfg.kcap)
    assert kout.item() == ref_k == 2
    assert np.array_equal(sel.cpu().numpy(), ref_sel)
    keep = [i for i in range(cfg.n_layers) if not ref_sel[i]]
    sub = ls.subset(keep)
    q.nf4_dequantize(sub, f, workspace(ls.ns, f))
    torch.cuda.synchronize()
    for i in keep:
        assert np.array_equal(np_of(ls.out_of(i), np.uint16), refs[i]["y"])
    for i in range(cfg.n_layers):
        if ref_sel[i]:   # promoted layers are not dequantised: output left untouched
            assert np.all(np_of(ls.out_of(i), np.uint8) == 0x5A)
    # the same step with the selection left on the device: the selected array
    # is the skip mask, no host round trip
    ls.out.view(torch.uint8).fill_(0x5A)
    q.nf4_dequantize_masked(ls, f, sel, workspace(ls.ns, f))
    torch.cuda.synchronize()
    for i in range(cfg.n_layers):
        if ref_sel[i]:
            assert np.all(np_of(ls.out_of(i), np.uint8) == 0x5A)
        else:
            assert np.array_equal(np_of(ls.out_of(i), np.uint16), refs[i]["y"])


@pytest.mark.parametrize("dq", [False, True], ids=["nodq", "dq"])
@pytest.mark.parametrize("dtname", ["bf16", "fp16"])
def test_masked_dequantize_matches_oracle(dtname, dq):
    """nf4_dequantize_masked on the edge layers (ragged sizes, zero, subnormal
    and huge blocks): the layers with a zero mask byte equal the oracle's
    dequantised values bit for bit, the others keep their poisoned output;
    an all-zero mask equals nf4_dequantize, an all-one mask writes nothing."""
    dtype = DTYPES[dtname]
    f = q.fmt(dtype, dq)
    layers = _edge_layers(dtype)
    print_case("masked dequant", dtname, "dq" if dq else "nodq", len(layers))
    ls = layerset([w for _, w in layers], f)
    layer_error(ls, f)
    ws = workspace(ls.ns, f)
    nl = len(layers)
    refs = [compare_layer(ls, i, w, dtype, dq) for i, (_, w) in enumerate(layers)]
    for pattern in ([i % 2 for i in range(nl)], [1 - i % 2 for i in range(nl)], [0] * nl, [1] * nl):
        skip = torch.tensor(pattern, dtype=torch.uint8, device="cuda")
        ls.out.view(torch.uint8).fill_(POISON)
        q.nf4_dequantize_masked(ls, f, skip, ws)
        torch.cuda.synchronize()
        for i in range(nl):
            if pattern[i]:
                assert np.all(np_of(ls.out_of(i), np.uint8) == POISON), (i, pattern)
            else:
                assert np.array_equal(np_of(ls.out_of(i), np.uint16), refs[i]["y"]), (i, pattern)


def test_single_matrix_with_outliers():
    cfg = configs.SINGLE
    f = q.fmt(cfg.dtype, cfg.dq)
    w = synth.generate(cfg, 0)
    print_case("single 4096x4096")
    ls = layerset([w], f)
    err = layer_error(ls, f)
    q.nf4_dequantize(ls, f, workspace(ls.ns, f))
    torch.cuda.synchronize()
    ref = compare_layer(ls, 0, w, cfg.dtype, cfg.dq, check_out=True)
    r = rel_err(err.item(), ref["err"])
    print(f"[single] err gpu {err.item():.12e} oracle {ref['err']:.12e} rel {r:.2e}", flush=True)
    assert r <= ERR_RTOL


def test_outputs_are_bitwise_deterministic():
    cfg = configs.SINGLE
    f = q.fmt(cfg.dtype, cfg.dq)
    w = synth.generate(cfg, 0)
    ls = layerset([w, w[:100_000]], f)
    ws = workspace(ls.ns, f)
    outs = []
    for rep in range(3):
        poison(ls)
        err = layer_error(ls, f, ws)
        q.nf4_dequantize(ls, f, ws)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (ls.codes, ls.absmax, ls.qabsmax, ls.scale2, ls.out)]
                    + [err.clone()])
    for rep in (1, 2):
        for a, b in zip(outs[0], outs[rep]):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_host_layer_array_may_be_reused_at_once():
    """The nf4_layer array is consumed before the call returns."""
    f = q.fmt(q.NF4_BF16, True)
    ws_list = [synth.generate_raw(40 + i, 16384 * (i + 1) + 3 * i) for i in range(6)]
    ls = layerset(ws_list, f)
    ws = workspace(ls.ns, f)
    err = torch.empty(len(ls), dtype=torch.float64, device="cuda")
    arr = (q.nf4_layer * len(ls))(*ls.c_layers)
    st = q.lib().nf4_layer_error(arr, len(ls), f, err.data_ptr(), ws.data_ptr(),
                                 ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == q.NF4_OK
    ctypes.memset(arr, 0xFF, ctypes.sizeof(arr))   # clobber right after the call
    torch.cuda.synchronize()
    for i, w in enumerate(ws_list):
        compare_layer(ls, i, w, q.NF4_BF16, True)


@pytest.mark.parametrize("call", ["nf4_quantize", "nf4_dequantize", "nf4_layer_error"])
def test_workspace_writes_stay_inside_the_minimum_size(call):
    """Each call given exactly the smallest workspace it accepts, followed by a
    guard region: the guard is untouched and the outputs are right."""
    f = q.fmt(q.NF4_BF16, True)
    ws_list = [synth.generate_raw(80 + i, n) for i, n in enumerate([16384 * 3 + 5, 100, 16384 * 7])]
    ls = layerset(ws_list, f)
    nl, ntiles = len(ls), sum((n + 16383) // 16384 for n in ls.ns)
    table = (nl * 64 + 255) // 256 * 256
    rec = (ntiles * 8 + 255) // 256 * 256      # the fused pass's 8-byte tile records
    part = (ntiles * 32 + 255) // 256 * 256    # fp64 partials / dequantisation records
    need = {"nf4_quantize": table + rec, "nf4_layer_error": table + rec + part,
            "nf4_dequantize": table + part}[call]
    guard = 4096
    buf = torch.full((need + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    err = torch.empty(nl, dtype=torch.float64, device="cuda")
    L, st = q.lib(), torch.cuda.current_stream().cuda_stream
    if call == "nf4_dequantize":   # codes and constants from a full-size workspace first
        q.nf4_layer_error(ls, f, err, workspace(ls.ns, f))
        torch.cuda.synchronize()
        ls.out.view(torch.uint8).fill_(0x5A)
    args = (ls.c_layers, nl, f)
    if call == "nf4_layer_error":
        assert L.nf4_layer_error(*args, err.data_ptr(), buf.data_ptr(), need - 1, st) == q.NF4_E_WORKSPACE
        rc = L.nf4_layer_error(*args, err.data_ptr(), buf.data_ptr(), need, st)
    else:
        assert getattr(L, call)(*args, buf.data_ptr(), need - 1, st) == q.NF4_E_WORKSPACE
        rc = getattr(L, call)(*args, buf.data_ptr(), need, st)
    assert rc == q.NF4_OK
    torch.cuda.synchronize()
    assert bool((buf[need:] == 0xA5).all())
    for i, w in enumerate(ws_list):
        compare_layer(ls, i, w, q.NF4_BF16, True, check_out=(call == "nf4_dequantize"))


# --------------------------------------------------------------------------
@pytest.mark.parametrize("nl", [1, 2, 7, 300, 1025, 4097, 65536])
def test_select_matches_oracle_on_the_same_scores(nl):
    rng = np.random.default_rng(nl)
    sws = torch.empty(q.aqlora_workspace_bytes(nl), dtype=torch.uint8, device="cuda")
    for trial in range(6):
        err = rng.random(nl)
        if trial % 2 == 0:
            err = np.round(err * 7) / 7          # many exact ties
        cost = rng.integers(1, 10**8, nl)
        if trial == 5:
            cost = rng.integers(-1000, 1000, nl)
        budget = [-1, 0, int(cost.sum() // 3), int(rng.integers(0, 10**9)), int(cost.sum()) * 2, 5][trial]
        kcap = [-1, -1, nl // 2, 3, -1, 0][trial]
        print_case("select", nl, trial)
        e = torch.from_numpy(err).cuda()
        c = torch.from_numpy(cost.astype(np.int64)).cuda()
        sel = torch.full((nl,), 7, dtype=torch.uint8, device="cuda")
        k = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        q.aqlora_select_topk(e, c, budget, kcap, sel, k, sws)
        torch.cuda.synchronize()
        rsel, rk = oracle.select_topk(err, cost, budget, kcap)
        assert k.item() == rk
        assert np.array_equal(sel.cpu().numpy(), rsel)
