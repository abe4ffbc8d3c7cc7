"""Pins for the oracle's codec variants (CPU only): block sizes 32/64/128/256
and the second-level kinds (none, int8, int8 with the mean absmax
subtracted, E4M3 8-bit float with the mean subtracted).

The pages say only that the constants are quantised again (QLoRA page, How
It Works, Double Quantization item; "QLoRA Explained", Double Quantization)
and fix 0.37 bit per parameter for the main reading.  Pins:
  * E4M3 decoding and nearest-even encoding equal torch's float8_e4m3fn
    conversion (a library routine), ties included;
  * block 64 with int8 (or none) is the main oracle, bit for bit;
  * other block sizes: absmax equals numpy's per-block maximum and codes the
    (separately pinned) encoder on fl32(x * fl32(1/a)) computed by numpy;
  * the mean is within one fp32 ulp of the exact rational mean; with equal
    absmax values the mean-offset kinds reconstruct a exactly;
  * the reconstructed constant is within half a step of the second level;
  * the bit accounting in closed form (the pages' 0.37 bit for block 64).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

BF16, FP16 = oracle.BF16, oracle.FP16
K0, K1, K2, K3 = oracle.KIND_NONE, oracle.KIND_INT8, oracle.KIND_INT8_MEAN, oracle.KIND_FP8_MEAN


def _torch_e4m3(vals):
    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_decode_equals_torch():
    codes = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.e4m3_decode(int(b)) for b in codes], np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_e4m3_encode_equals_torch_including_ties():
    mags = sorted({oracle.e4m3_decode(b) for b in range(0x7F)})
    mids = [(a + b) / 2 for a, b in zip(mags[:-1], mags[1:])]           # exact ties
    rng = np.random.default_rng(0)
    vals = np.r_[mags, mids, rng.uniform(0, 448, 3000), rng.uniform(0, 2.0 ** -5, 2000)]
    vals = np.r_[vals, -vals].astype(np.float32)
    got = np.array([oracle.e4m3_encode(float(v)) for v in vals], np.uint8)
    ref = _torch_e4m3(vals)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dtype", [BF16, FP16])
@pytest.mark.parametrize("kind", [K0, K1])
def test_block64_is_the_main_codec(dtype, kind):
    w = synth.generate_raw(123, 64 * 256 * 3 + 77, dtype=dtype, outlier_frac=0.003)
    a = oracle.layer_error_ex(w, dtype, 64, kind)
    b = oracle.layer_error(w, dtype, kind == K1)
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["absmax"].view(np.uint32), b["absmax"].view(np.uint32))
    assert np.array_equal(a["y"], b["y"]) and a["err"] == b["err"]
    if kind == K1:
        assert np.array_equal(a["q"].view(np.int8), b["qabsmax"])
        assert np.array_equal(a["scale2"].view(np.uint32), b["scale2"].view(np.uint32))


@pytest.mark.parametrize("block", [32, 128, 256])
def test_other_block_sizes_group_and_encode(block):
    dtype = BF16
    w = synth.generate_raw(200 + block, block * 300 + 13, dtype=dtype, outlier_frac=0.002)
    w[block * 7: block * 8] = 0                                      # a zero block
    r = oracle.layer_error_ex(w, dtype, block, K0)
    x = oracle.from16(w, dtype)
    nb = (x.size + block - 1) // block
    pad = np.zeros(nb * block, np.float32)
    pad[:x.size] = np.abs(x)
    amax = pad.reshape(nb, block).max(axis=1)
    assert np.array_equal(r["absmax"].view(np.uint32), amax.view(np.uint32))
    a = np.repeat(amax, block)[:x.size]
    nz = a > 0
    s = np.zeros_like(x)
    s[nz] = x[nz] * (np.float32(1) / a[nz])                          # fl32(x * fl32(1/a))
    exp = oracle.encode(s)
    exp[~nz] = 7
    codes = np.empty(x.size, np.uint8)
    codes[0::2] = r["codes"] & 15
    codes[1::2] = (r["codes"] >> 4)[: x.size // 2]
    assert np.array_equal(codes, exp)


@pytest.mark.parametrize("kind", [K2, K3])
def test_mean_and_constant_absmax(kind):
    w = synth.generate_raw(300, 64 * 700 + 5, dtype=BF16, outlier_frac=0.002)
    r = oracle.layer_error_ex(w, BF16, 64, kind)
    exact = sum(Fraction(float(v)) for v in r["absmax"]) / r["absmax"].size
    mu = np.float32(r["mean"])
    ulp = np.spacing(mu)
    assert abs(Fraction(float(mu)) - exact) <= Fraction(float(ulp))
    # equal absmax everywhere: every c is 0, q is 0, a' = mu = a exactly -> same y as no DQ
    rng = np.random.default_rng(1)
    v = rng.integers(0x3D00, 0x3E00, 64 * 600).astype(np.uint16)
    v[::64] = 0x3E80                                                 # every block's max: 0.25
    a = oracle.layer_error_ex(v, BF16, 64, kind)
    b = oracle.layer_error_ex(v, BF16, 64, K0)
    assert a["mean"] == 0.25 and not a["q"].any() and not a["scale2"].any()
    assert np.array_equal(a["y"], b["y"]) and a["err"] == b["err"]


@pytest.mark.parametrize("kind", [K1, K2, K3])
def test_reconstructed_constant_within_half_a_step(kind):
    w = synth.generate_raw(400 + kind, 64 * 256 * 4, dtype=BF16, outlier_frac=0.005)
    r = oracle.layer_error_ex(w, BF16, 64, kind)
    a = r["absmax"].astype(np.float64)
    mu = r["mean"] if kind != K1 else 0.0
    s2 = np.repeat(r["scale2"].astype(np.float64), 256)[: a.size]
    if kind == K3:
        qv = np.array([oracle.e4m3_decode(int(b)) for b in r["q"]], np.float64)
        c = a - mu
        # E4M3 spacing at |c/s2|: 2^(floor(log2 v) - 3) for normal values, 2^-9 below 2^-6
        v = np.where(s2 > 0, np.abs(c) / np.where(s2 > 0, s2, 1.0), 0.0)
        e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
        step = 2.0 ** (e - 3) * s2
        rec = qv * s2 + mu
        assert np.all(np.abs(rec - a) <= 0.5 * step * (1 + 1e-6) + 1e-6 * np.abs(a))
    else:
        qv = r["q"].view(np.int8).astype(np.float64)
        rec = qv * s2 + mu
        assert np.all(np.abs(rec - a) <= 0.5 * s2 * (1 + 1e-5) + 1e-6 * np.abs(a))


def test_bit_accounting():
    n = 4096 * 4096
    # bits per parameter spent on constants, and what the second level saves
    for block in (32, 64, 128, 256):
        b0 = 8 * (oracle.storage_bytes_ex(n, block, K0) - n // 2) / n
        b1 = 8 * (oracle.storage_bytes_ex(n, block, K1) - n // 2) / n
        assert b0 == 32 / block
        assert b1 == 8 / block + 32 / (block * 256)
    saved64 = 8 * (oracle.storage_bytes_ex(n, 64, K0) - oracle.storage_bytes_ex(n, 64, K1)) / n
    assert saved64 == 0.373046875 and round(saved64, 2) == 0.37     # the pages' figure
    # the mean costs one fp32 per matrix
    for k in (K2, K3):
        assert oracle.storage_bytes_ex(n, 64, k) == oracle.storage_bytes_ex(n, 64, K1) + 4


@pytest.mark.parametrize("block", [32, 128])
@pytest.mark.parametrize("kind", [K1, K2, K3])
def test_group_maximum_takes_the_top_code(block, kind):
    """In every group with a nonzero |c| maximum, the block holding it maps to
    the second level's largest value: 127 for the int8 kinds, 448 for E4M3
    (so s2 is that maximum over 127 or 448, not some other divisor), and
    every other block stays within it."""
    w = synth.generate_raw(900 + kind + block, block * 256 * 5 + 3 * block + 7, dtype=BF16,
                           outlier_frac=0.003)
    r = oracle.layer_error_ex(w, BF16, block, kind)
    a = r["absmax"].astype(np.float64)
    c = a - (r["mean"] if kind != K1 else 0.0)
    if kind == K3:
        qv = np.array([oracle.e4m3_decode(int(b)) for b in r["q"]], np.float64)
        top = 448.0
    else:
        qv = r["q"].view(np.int8).astype(np.float64)
        top = 127.0
    ng = r["scale2"].size
    for g in range(ng):
        sl = slice(256 * g, min(256 * (g + 1), a.size))
        cg, qg = np.abs(c[sl]), np.abs(qv[sl])
        if cg.max() == 0:
            assert r["scale2"][g] == 0 and not qg.any()
            continue
        assert qg[int(np.argmax(cg))] == top, g
        assert qg.max() == top, g
        assert r["scale2"][g] == np.float32(np.float32(cg.max()) / np.float32(top)), g
