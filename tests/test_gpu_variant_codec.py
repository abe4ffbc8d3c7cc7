"""GPU parity of the codec variants (block 32/64/128/256 x second-level kind
none / int8 / int8 minus the mean / E4M3 minus the mean) against the oracle.

Codes, absmax, the second-level byte, scales, the mean and the dequantised
values bit-exact; errors within 1e-12 relative (both sum exact squares in
fp64, in different orders).  Ragged sizes around every block and group
boundary, a zero matrix, tiny and huge values, outliers; bf16, and fp16 for
the main block sizes; the 14B stack's attention and FFN shapes whole.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_lora_fine_nf4_amd as q
import synth
from conftest import print_case
from gpu_util import poison

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    q.lib()
    yield
    torch.cuda.synchronize()


def _layers(dtype, block):
    g = 256 * block
    L = [synth.generate_raw(1000 + k, n, dtype=dtype, outlier_frac=0.003)
         for k, n in enumerate([1, block - 1, block, block + 1, 1000, g - 1, g, g + 1,
                                3 * g + 77])]
    L.append(np.zeros(g + block, np.uint16))
    rng = np.random.default_rng(block + dtype)
    if dtype == q.NF4_BF16:
        e = rng.integers(0x0A00, 0x0D00, block * 40).astype(np.uint16)      # absmax < 2^-100
        e |= (rng.integers(0, 2, e.size).astype(np.uint16) << 15)
        L.append(e)
        h = rng.integers(0x7E00, 0x7F7F, block * 40).astype(np.uint16)      # up to 3.4e38
        L.append(h)
    return L


def _run(ws_list, dtype, block, kind):
    v = q.variant(dtype, block, kind)
    f = q.fmt(dtype, kind != q.NF4_DQ_NONE)
    ls = q.LayerSet([w.size for w in ws_list], f, with_absmax=True, block=block)
    for i, w in enumerate(ws_list):
        ls.w_of(i).copy_(torch.from_numpy(np.ascontiguousarray(w, np.uint16).view(np.int16)))
    poison(ls)
    nl = len(ws_list)
    ws = torch.empty(q.nf4_workspace_bytes_variant(ls.ns, v), dtype=torch.uint8, device="cuda")
    err = torch.full((nl,), float("nan"), dtype=torch.float64, device="cuda")
    mean = torch.full((nl,), float("nan"), dtype=torch.float32, device="cuda")
    q.nf4_layer_error_variant(ls, v, err, ws, mean=mean)
    q.nf4_dequantize_variant(ls, v, ws, mean=mean)
    torch.cuda.synchronize()
    return ls, err.cpu().numpy(), mean.cpu().numpy()


def _compare(ls, errs, means, ws_list, dtype, block, kind):
    for i, w in enumerate(ws_list):
        ref = oracle.layer_error_ex(w, dtype, block, kind)
        tag = (i, w.size)
        assert np.array_equal(ls.codes_of(i).cpu().numpy(), ref["codes"]), tag
        assert np.array_equal(ls.absmax_of(i).cpu().numpy().view(np.uint32),
                              ref["absmax"].view(np.uint32)), tag
        if kind != q.NF4_DQ_NONE:
            assert np.array_equal(ls.qabsmax_of(i).cpu().numpy().view(np.uint8), ref["q"]), tag
            assert np.array_equal(ls.scale2_of(i).cpu().numpy().view(np.uint32),
                                  ref["scale2"].view(np.uint32)), tag
        if kind >= q.NF4_DQ_INT8_MEAN:
            assert np.float32(means[i]).view(np.uint32) == np.float32(ref["mean"]).view(np.uint32), tag
        assert np.array_equal(ls.out_of(i).cpu().numpy().view(np.uint16), ref["y"]), tag
        r = ref["err"]
        assert (errs[i] == r == 0.0) or abs(errs[i] - r) <= 1e-12 * r, (tag, errs[i], r)


@pytest.mark.parametrize("kind", [0, 1, 2, 3], ids=["none", "int8", "int8mean", "e4m3mean"])
@pytest.mark.parametrize("block", [32, 64, 128, 256])
def test_variant_bf16(block, kind):
    print_case("variant", "bf16", block, kind)
    ws_list = _layers(q.NF4_BF16, block)
    ls, errs, means = _run(ws_list, q.NF4_BF16, block, kind)
    _compare(ls, errs, means, ws_list, q.NF4_BF16, block, kind)


@pytest.mark.parametrize("kind", [1, 3], ids=["int8", "e4m3mean"])
@pytest.mark.parametrize("block", [32, 128])
def test_variant_fp16(block, kind):
    print_case("variant", "fp16", block, kind)
    ws_list = _layers(q.NF4_FP16, block)
    ls, errs, means = _run(ws_list, q.NF4_FP16, block, kind)
    _compare(ls, errs, means, ws_list, q.NF4_FP16, block, kind)


def test_block64_int8_variant_equals_the_main_codec():
    """The variant path at block 64 with int8 is the fused main codec's output."""
    ws_list = _layers(q.NF4_BF16, 64)
    ls, errs, _ = _run(ws_list, q.NF4_BF16, 64, 1)
    f = q.fmt(q.NF4_BF16, True)
    ls2 = q.LayerSet([w.size for w in ws_list], f, with_absmax=True)
    ls2.w.copy_(ls.w)
    ws = torch.empty(q.nf4_workspace_bytes(ls2.ns, f), dtype=torch.uint8, device="cuda")
    err2 = torch.empty(len(ws_list), dtype=torch.float64, device="cuda")
    q.nf4_layer_error(ls2, f, err2, ws)
    q.nf4_dequantize(ls2, f, ws)
    torch.cuda.synchronize()
    for i in range(len(ws_list)):
        assert torch.equal(ls.codes_of(i), ls2.codes_of(i))
        assert torch.equal(ls.qabsmax_of(i), ls2.qabsmax_of(i))
        assert torch.equal(ls.out_of(i), ls2.out_of(i))
    e2 = err2.cpu().numpy()
    assert np.all(np.abs(errs - e2) <= 1e-5 * np.maximum(e2, 1e-300))


@pytest.mark.slow
@pytest.mark.parametrize("block,kind", [(128, 3), (32, 2)])
def test_variant_fullsize_matrices(block, kind):
    from synth import configs
    cfg = configs.BY_NAME["14b"]
    idx = [0, 5, 6]                                    # q, up, down of block 0
    ws_list = [synth.generate(cfg, i, threads=8) for i in idx]
    print_case("variant full size", block, kind, [w.size for w in ws_list])
    ls, errs, means = _run(ws_list, cfg.dtype, block, kind)
    _compare(ls, errs, means, ws_list, cfg.dtype, block, kind)
