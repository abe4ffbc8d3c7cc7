"""One matrix of more than 2^31 weights (element indices past 2^31, byte
offsets past 4 GiB, a ragged last block and tile): the fused pass, the
dequantisation and the codec variants.

Sampled tiles (the first, the two on either side of element 2^31, the
ragged last one) bit-exact against the oracle on the same slice (a tile is
one double-quant group, so its outputs depend on its own weights only);
the error against an fp64 sum of the device's own weights and dequantised
values; the variants' groups likewise (kinds without the mean), and the
variant mean against a sequential fp64 sum (numpy cumsum) of the device's
absmax values in block and group order.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_lora_fine_nf4_amd as q
import synth
from conftest import print_case

pytestmark = pytest.mark.gpu
BF16 = q.NF4_BF16
N = (1 << 31) + 12_347          # not a multiple of 64 or of 16384
TILE = 16384


@pytest.fixture(scope="module")
def big():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    q.lib()
    print_case("large matrix", N)
    w = synth.generate_raw(4242, N, outlier_frac=1e-4, threads=16)
    f = q.fmt(BF16, True)
    ls = q.LayerSet([N], f, with_absmax=True)
    ls.w_of(0).copy_(torch.from_numpy(w.view(np.int16)))
    yield w, ls
    del ls
    torch.cuda.empty_cache()


def _dev_sse(ls):
    """sum of (x - y)^2 over the matrix, fp64 on the device, in chunks"""
    x, y = ls.w_of(0), ls.out_of(0)
    s = 0.0
    for c in range(0, N, 1 << 28):
        xs = x[c:c + (1 << 28)].view(torch.bfloat16).double()
        ys = y[c:c + (1 << 28)].view(torch.bfloat16).double()
        s += float(((xs - ys) ** 2).sum())
    return s


def test_fused_pass_and_dequant_past_2g(big):
    w, ls = big
    f = q.fmt(BF16, True)
    ws = torch.empty(q.nf4_workspace_bytes(ls.ns, f), dtype=torch.uint8, device="cuda")
    err = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    q.nf4_layer_error(ls, f, err, ws)
    q.nf4_dequantize(ls, f, ws)
    torch.cuda.synchronize()
    last = (N - 1) // TILE
    t2g = (1 << 31) // TILE
    for t in sorted({0, t2g - 1, t2g, last}):
        e0, e1 = t * TILE, min((t + 1) * TILE, N)
        ref = oracle.layer_error(w[e0:e1], BF16, True)
        print_case("tile", t, e0, e1)
        c0 = e0 // 2
        assert np.array_equal(ls.codes_of(0)[c0:c0 + ref["codes"].size].cpu().numpy(), ref["codes"]), t
        b0 = e0 // 64
        assert np.array_equal(ls.absmax_of(0)[b0:b0 + ref["absmax"].size].cpu().numpy().view(np.uint32),
                              ref["absmax"].view(np.uint32)), t
        assert np.array_equal(ls.qabsmax_of(0)[b0:b0 + ref["qabsmax"].size].cpu().numpy(), ref["qabsmax"]), t
        assert np.float32(ls.scale2_of(0)[t].item()).view(np.uint32) == ref["scale2"].view(np.uint32)[0], t
        assert np.array_equal(ls.out_of(0)[e0:e1].cpu().numpy().view(np.uint16), ref["y"]), t
    e, r = err.item(), _dev_sse(ls)
    assert abs(e - r) <= 1e-5 * r, (e, r)


@pytest.mark.parametrize("block,kind", [(32, 1), (256, 0), (32, 2)])
def test_variants_past_2g(big, block, kind):
    w, ls = big
    print_case("large matrix variant", block, kind)
    v = q.variant(BF16, block, kind)
    vs = q.LayerSet([N], q.fmt(BF16, kind != 0), with_absmax=True, w=ls.w, codes=ls.codes,
                    out=ls.out, block=block)
    ws = torch.empty(q.nf4_workspace_bytes_variant(vs.ns, v), dtype=torch.uint8, device="cuda")
    err = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    mean = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    q.nf4_layer_error_variant(vs, v, err, ws, mean=mean)
    q.nf4_dequantize_variant(vs, v, ws, mean=mean)
    torch.cuda.synchronize()
    G = 256 * block
    nb = (N + block - 1) // block
    if kind >= 2:
        a = vs.absmax_of(0).cpu().numpy().astype(np.float64)
        ng = (nb + 255) // 256
        pad = np.zeros(ng * 256)
        pad[:nb] = a
        gs = np.cumsum(pad.reshape(ng, 256), axis=1)[:, -1]      # each group, block order
        S = np.cumsum(gs)[-1]                                     # groups in order
        mu = np.float32(S / nb)
        assert mu.view(np.uint32) == np.float32(mean.item()).view(np.uint32)
    else:
        last = (N - 1) // G
        g2g = (1 << 31) // G
        for g in sorted({0, g2g - 1, g2g, last}):
            e0, e1 = g * G, min((g + 1) * G, N)
            ref = oracle.layer_error_ex(w[e0:e1], BF16, block, kind)
            c0, b0 = e0 // 2, e0 // block
            assert np.array_equal(vs.codes_of(0)[c0:c0 + ref["codes"].size].cpu().numpy(), ref["codes"]), g
            assert np.array_equal(vs.absmax_of(0)[b0:b0 + ref["absmax"].size].cpu().numpy().view(np.uint32),
                                  ref["absmax"].view(np.uint32)), g
            if kind == 1:
                assert np.array_equal(vs.qabsmax_of(0)[b0:b0 + ref["q"].size].cpu().numpy().view(np.uint8),
                                      ref["q"]), g
                assert (np.float32(vs.scale2_of(0)[g].item()).view(np.uint32)
                        == ref["scale2"].view(np.uint32)[0]), g
            assert np.array_equal(vs.out_of(0)[e0:e1].cpu().numpy().view(np.uint16), ref["y"]), g
    e, r = err.item(), _dev_sse(vs)
    assert abs(e - r) <= 1e-9 * r, (e, r)
