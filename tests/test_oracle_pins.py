"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: a library normal
quantile, a library float conversion, exact rational nearest-level search,
closed forms of the byte accounting, figures the pages print, and properties
the method must have.  A plausible mistake anywhere in the oracle (a wrong
level, a threshold rounded the wrong way, a swapped nibble, a dropped
double-quant term, a wrong sign in the ranking) fails at least one of them.
"""
import json
import math
import os
import statistics
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy import special, stats

import oracle
import synth
from synth import configs

DELTA = 929 / 960


# --------------------------------------------------------------------------
# O1 levels
# --------------------------------------------------------------------------
def test_level_count_matches_pages(golden_dir):
    figs = json.load(open(os.path.join(golden_dir, "pages_figures.json")))
    v = oracle.levels()
    assert v.size == figs["nf4_level_count"]["value"]


def test_levels_exact_zero_and_unit_endpoints_strictly_ascending():
    v = oracle.levels()
    assert v[0] == -1.0 and v[15] == 1.0 and v[7] == 0.0
    assert not np.signbit(v[7])
    assert np.all(np.diff(v.astype(np.float64)) > 0)
    assert np.sum(v < 0) == 7 and np.sum(v > 0) == 8


@pytest.mark.parametrize("ppf", ["scipy_ndtri", "statistics_inv_cdf"])
def test_levels_equal_library_normal_quantiles(ppf):
    """Rebuild the quantile levels with library inverse-normal routines."""
    f = special.ndtri if ppf == "scipy_ndtri" else statistics.NormalDist().inv_cdf
    top = float(f(DELTA))
    neg = [-float(f(DELTA - k * (DELTA - 0.5) / 7)) / top for k in range(7)]
    pos = [float(f(DELTA - k * (DELTA - 0.5) / 8)) / top for k in range(8)][::-1]
    ref = np.array(neg + [0.0] + pos, np.float64).astype(np.float32)
    assert np.array_equal(ref.view(np.uint32), oracle.levels().view(np.uint32))


def test_levels_sit_at_evenly_spaced_probabilities():
    """Each level is a normal quantile: Phi(level * z_delta) steps evenly."""
    v = oracle.levels().astype(np.float64)
    z = special.ndtri(DELTA)
    p = stats.norm.cdf(v * z)
    pos = p[7:]                       # 0.5 .. delta over codes 7..15
    neg = p[:8]                       # 1-delta .. 0.5 over codes 0..7
    assert np.allclose(np.diff(pos), (DELTA - 0.5) / 8, atol=2e-7)
    assert np.allclose(np.diff(neg), (DELTA - 0.5) / 7, atol=2e-7)
    assert abs(p[15] - DELTA) < 1e-7 and abs(p[0] - (1 - DELTA)) < 1e-7


# --------------------------------------------------------------------------
# O2 / O5 thresholds and encode == nearest level
# --------------------------------------------------------------------------
def _nearest_exact(s: Fraction, levels) -> int:
    """Exact nearest level, ties to the lower code (brute force)."""
    best, bd = 0, None
    for i, lv in enumerate(levels):
        d = abs(s - lv)
        if bd is None or d < bd:
            best, bd = i, d
    return best


def test_thresholds_are_midpoints_rounded_down():
    v = [Fraction(float(x)) for x in oracle.levels()]
    t = oracle.thresholds()
    for i in range(15):
        mid = (v[i] + v[i + 1]) / 2
        ti = Fraction(float(t[i]))
        nxt = Fraction(float(np.nextafter(t[i], np.float32(np.inf))))
        assert ti <= mid < nxt


def test_encode_equals_exact_nearest_level_on_all_fp32():
    """Both rules are monotone step functions of s, so they agree on every
    fp32 value iff they agree on both sides of every step of either rule."""
    levels = [Fraction(float(x)) for x in oracle.levels()]
    t = oracle.thresholds()
    probes = []
    for i in range(15):
        probes += [t[i], np.nextafter(t[i], np.float32(np.inf)),
                   np.nextafter(t[i], np.float32(-np.inf))]
    probes += [np.float32(x) for x in (-1.0001, -1.0, 0.0, -0.0, 1.0, 1.0001, 3.0, -3.0)]
    probes = np.array(probes, np.float32)
    codes = oracle.encode(probes)
    for s, c in zip(probes, codes):
        assert c == _nearest_exact(Fraction(float(s)), levels), float(s)
    # step positions of the exact rule: between the probe pairs around each t_i
    for i in range(15):
        assert oracle.encode(np.array([t[i]], np.float32))[0] == i
        assert oracle.encode(np.array([np.nextafter(t[i], np.float32(np.inf))], np.float32))[0] == i + 1


def test_encode_vs_bruteforce_random_and_monotone():
    rng = np.random.default_rng(1)
    s = rng.uniform(-1.0001, 1.0001, 200_000).astype(np.float32)
    s = np.concatenate([s, (rng.standard_normal(50_000) * 0.3).astype(np.float32)])
    codes = oracle.encode(s)
    v = oracle.levels().astype(np.float64)
    dist = np.abs(s.astype(np.float64)[:, None] - v[None, :])
    ref = np.argmin(dist, axis=1)  # argmin picks the first (lower) index on ties
    assert np.array_equal(codes, ref.astype(np.uint8))
    order = np.argsort(s, kind="stable")
    assert np.all(np.diff(codes[order].astype(int)) >= 0)


# --------------------------------------------------------------------------
# 16-bit rounding
# --------------------------------------------------------------------------
def _special_f32():
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.996, 65520.0, 65536.0, 1e-45, 2**-149,
            2**-126, 2**-127 * 3, 2**-133, 2**-134, 2**-24, 2**-25, 2**-25 * 3, 2**-14,
            3.3895314e38, 3.4e38, 6e-8, 5.96e-8, 1.0009765625, 1.00048828125]
    return np.array(vals + [-x for x in vals], np.float32)


def test_to_bf16_rne_matches_torch():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2**32, 400_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    # ties: low 16 bits exactly 0x8000
    ties = ((rng.integers(0, 2**16, 20_000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    f = np.concatenate([f, ties, _special_f32()]).astype(np.float32)
    ours = oracle.to16_rne(f, oracle.BF16)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_to_fp16_rne_matches_numpy():
    rng = np.random.default_rng(3)
    f = np.concatenate([
        (rng.standard_normal(300_000) * 0.05).astype(np.float32),
        rng.uniform(-70000, 70000, 50_000).astype(np.float32),
        (rng.uniform(-1, 1, 50_000) * 2.0**-14).astype(np.float32),
        # fp16 ties: fp32 values halfway between two fp16 values
        (np.arange(2048, 4096, dtype=np.float32) + 0.5) * np.float32(2.0**-11),
        _special_f32()]).astype(np.float32)
    ours = oracle.to16_rne(f, oracle.FP16)
    with np.errstate(over="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_from16_exact():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = (h & 0x7F80) != 0x7F80
    bf = oracle.from16(h, oracle.BF16)
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(bf[fin].view(np.uint32), ref[fin].view(np.uint32))
    fin16 = (h & 0x7C00) != 0x7C00
    fp = np.array([oracle.lib().nf4o_from16(int(x), 1) for x in h[fin16][::97]], np.float32)
    assert np.array_equal(fp, h[fin16][::97].view(np.float16).astype(np.float32))


# --------------------------------------------------------------------------
# O3-O6 quantise: codes against exact nearest on tiny inputs, layout, zeros
# --------------------------------------------------------------------------
def _codes_unpacked(codes, n):
    lo = codes & 15
    hi = codes >> 4
    out = np.empty(2 * codes.size, np.uint8)
    out[0::2], out[1::2] = lo, hi
    return out[:n]


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_quantize_codes_are_nearest_level_of_x_over_absmax(dtype):
    w = synth.generate_raw(11 + dtype, 64 * 24 + 37, dtype=dtype, outlier_frac=0.01)
    n = w.size
    codes, absmax = oracle.quantize(w, dtype)
    x = oracle.from16(w, dtype)
    c = _codes_unpacked(codes, n)
    levels = [Fraction(float(t)) for t in oracle.levels()]
    mids = [(levels[i] + levels[i + 1]) / 2 for i in range(15)]
    near_tie = 0
    for b in range((n + 63) // 64):
        blk = x[64 * b: 64 * b + 64]
        a = max(abs(Fraction(float(t))) for t in blk)
        assert Fraction(float(absmax[b])) == a
        for j, xv in enumerate(blk):
            i = 64 * b + j
            s_exact = Fraction(float(xv)) / a
            # the reading normalises as x * fl32(1/a): identical nearest level
            # except within a few ulps of a midpoint
            s_read = Fraction(float(np.float32(xv) * (np.float32(1) / np.float32(float(a)))))
            assert c[i] == _nearest_exact(s_read, levels)
            ref = _nearest_exact(s_exact, levels)
            if c[i] != ref:
                near_tie += 1
                assert abs(int(c[i]) - ref) == 1
                assert min(abs(s_exact - m) for m in mids) < Fraction(1, 2**21)
    assert near_tie <= 2


def test_pack_layout_low_nibble_first_and_odd_tail():
    a = 2.0 ** -3
    v = oracle.levels()
    vals = oracle.to16_rne((v * np.float32(a)).astype(np.float32), oracle.BF16)
    # 16 values in code order, then reversed, then one extra -> odd n = 33
    w = np.concatenate([vals, vals[::-1], vals[3:4]]).astype(np.uint16)
    codes, absmax = oracle.quantize(w, oracle.BF16)
    assert absmax[0] == np.float32(a)
    assert codes.size == 17
    expect = list(range(16)) + list(range(15, -1, -1)) + [3]
    for j in range(16):
        assert codes[j] == (expect[2 * j] | (expect[2 * j + 1] << 4))
    assert codes[16] == 3  # high nibble of the odd tail is zero


@pytest.mark.parametrize("dq", [False, True])
def test_zero_block_maps_to_zero(dq):
    w = np.zeros(64 * 5 + 10, np.uint16)
    w[70] = 0x8000  # -0.0
    r = oracle.layer_error(w, oracle.BF16, dq)
    assert np.all(r["codes"][:-1] == 0x77) and r["codes"][-1] == 0x77
    assert np.all(r["absmax"] == 0)
    assert np.all(r["y"] == 0)           # +0, never -0
    assert r["err"] == 0.0
    if dq:
        assert np.all(r["qabsmax"] == 0) and np.all(r["scale2"] == 0)


def test_subnormal_absmax_block_is_encoded_by_nearest_level():
    # a bf16 block whose largest |x| is subnormal: the 2^64 prescale path
    levels = [Fraction(float(t)) for t in oracle.levels()]
    w = np.array([1, 2, 3, 0x8005, 0x8007, 0x0004, 0, 0x8000] * 8, np.uint16)
    codes, absmax = oracle.quantize(w, oracle.BF16)
    x = oracle.from16(w, oracle.BF16)
    a = Fraction(float(absmax[0]))
    assert absmax[0] == np.float32(7 * 2.0 ** -133)
    c = _codes_unpacked(codes, w.size)
    for i, xv in enumerate(x):
        assert c[i] == _nearest_exact(Fraction(float(xv)) / a, levels)


# --------------------------------------------------------------------------
# O7 double quantisation
# --------------------------------------------------------------------------
def test_double_quant_properties():
    w = synth.generate_raw(21, 64 * 256 * 3 + 64 * 17, outlier_frac=0.001)
    codes, absmax = oracle.quantize(w, oracle.BF16)
    q, s2 = oracle.double_quant(absmax)
    nb = absmax.size
    assert s2.size == 4
    for g in range(s2.size):
        blk = absmax[256 * g: 256 * g + 256]
        G = blk.max()
        assert s2[g] == np.float32(G) / np.float32(127)
        qb = q[256 * g: 256 * g + 256].astype(np.int64)
        assert qb[np.argmax(blk)] == 127
        assert np.all((qb >= 0) & (qb <= 127))
        ad = qb.astype(np.float32) * s2[g]
        assert np.all(np.abs(ad.astype(np.float64) - blk) <= 0.5 * float(s2[g]) * (1 + 2**-20))
    assert q.size == nb


def test_double_quant_saving_matches_pages_figure(golden_dir):
    figs = json.load(open(os.path.join(golden_dir, "pages_figures.json")))
    stated = figs["double_quant_saving_bits_per_param"]["value"]
    n = 4096 * 4096
    saved_bits = (oracle.storage_bytes(n, False) - oracle.storage_bytes(n, True)) * 8 / n
    assert saved_bits == 0.373046875            # 32/64 - (8/64 + 32/16384)
    assert round(saved_bits, 2) == stated
    assert oracle.storage_bytes(n, False) == 9_437_184
    assert oracle.storage_bytes(n, True) == 8_654_848


# --------------------------------------------------------------------------
# O8 dequantisation invariants
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
@pytest.mark.parametrize("dq", [False, True])
def test_dequant_outputs_lie_in_block_level_table(dtype, dq):
    w = synth.generate_raw(31, 64 * 300 + 5, dtype=dtype, outlier_frac=0.002)
    r = oracle.layer_error(w, dtype, dq)
    v = oracle.levels()
    c = _codes_unpacked(r["codes"], w.size)
    for b in range((w.size + 63) // 64):
        ad = (np.float32(r["qabsmax"][b]) * r["scale2"][b // 256]) if dq else r["absmax"][b]
        table = oracle.to16_rne((v * np.float32(ad)).astype(np.float32), dtype)
        sl = slice(64 * b, 64 * b + 64)
        assert np.array_equal(r["y"][sl], table[c[sl]])


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_level_values_decode_to_their_codes(dtype):
    v = oracle.levels()
    for k in (-6, -3, 0, 2):
        a = np.float32(2.0 ** k)
        vals = oracle.to16_rne((v * a).astype(np.float32), dtype)
        codes, absmax = oracle.quantize(np.tile(vals, 4), dtype)
        assert absmax[0] == a
        assert np.array_equal(_codes_unpacked(codes, 64), np.tile(np.arange(16), 4))
        y = oracle.dequantize(codes, 64, dtype, absmax=absmax)
        assert np.array_equal(y, np.tile(vals, 4))


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_requantising_the_dequantised_matrix_is_idempotent(dtype):
    w = synth.generate_raw(41, 64 * 500, dtype=dtype)
    codes, absmax = oracle.quantize(w, dtype)
    y = oracle.dequantize(codes, w.size, dtype, absmax=absmax)
    codes2, absmax2 = oracle.quantize(y, dtype)
    assert np.array_equal(absmax2.view(np.uint32), absmax.view(np.uint32))
    assert np.array_equal(codes2, codes)


# --------------------------------------------------------------------------
# O9 error
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_error_is_zero_for_a_matrix_of_levels(dtype):
    v = oracle.levels()
    vals = oracle.to16_rne((v * np.float32(0.25)).astype(np.float32), dtype)
    r = oracle.layer_error(np.tile(vals, 40), dtype, False)
    assert r["err"] == 0.0


@pytest.mark.parametrize("dq", [False, True])
def test_error_equals_exact_rational_sum(dq):
    w = synth.generate_raw(51, 64 * 40 + 3, outlier_frac=0.01)
    r = oracle.layer_error(w, oracle.BF16, dq)
    x = oracle.from16(w, oracle.BF16)
    y = oracle.from16(r["y"], oracle.BF16)
    exact = sum((Fraction(float(a)) - Fraction(float(b))) ** 2 for a, b in zip(x, y))
    assert r["err"] == float(exact)


# --------------------------------------------------------------------------
# O10 / O11 cost and selection
# --------------------------------------------------------------------------
def test_promotion_cost_closed_forms():
    # per-matrix costs of the stacks (2n - NF4 bytes)
    assert oracle.promote_cost(65536, False) == 94_208
    assert oracle.promote_cost(176_128, False) == 253_184
    assert oracle.promote_cost(12_582_912, True) == 18_674_688
    assert oracle.promote_cost(16_777_216, True) == 24_899_584
    assert oracle.promote_cost(45_088_768, True) == 66_917_632
    assert oracle.promote_cost(26_214_400, True) == 38_905_600
    assert oracle.promote_cost(70_778_880, True) == 105_045_120
    # tails: odd n, partial block, partial group
    n = 64 * 256 + 65
    assert oracle.storage_bytes(n, True) == (n + 1) // 2 + 258 + 4 * 2
    assert oracle.storage_bytes(n, False) == (n + 1) // 2 + 4 * 258


def _select_by_sorted(err, cost, budget, kcap):
    order = sorted(range(len(err)), key=lambda i: (-err[i], i))
    K, tot = 0, 0
    for i in order:
        if kcap >= 0 and K >= kcap:
            break
        if budget >= 0 and tot + cost[i] > budget:
            break
        tot += cost[i]
        K += 1
    sel = np.zeros(len(err), np.uint8)
    sel[order[:K]] = 1
    return sel, K


def test_selection_reduces_to_library_sort_and_prefix():
    rng = np.random.default_rng(7)
    for trial in range(200):
        nl = int(rng.integers(1, 60))
        err = rng.choice([0.5, 1.0, 2.0, 3.5], nl) if trial % 3 == 0 else rng.random(nl)
        cost = rng.integers(-5, 100, nl)
        budget = int(rng.integers(-1, 1500))
        kcap = int(rng.integers(-1, nl + 2))
        sel, K = oracle.select_topk(err, cost, budget, kcap)
        rsel, rK = _select_by_sorted(list(err), list(cost), budget, kcap)
        assert K == rK and np.array_equal(sel, rsel)


def test_selection_monotone_in_budget_and_error():
    cfg = configs.TOY
    errs = []
    for i in range(cfg.n_layers):
        errs.append(oracle.layer_error(synth.generate(cfg, i), cfg.dtype, cfg.dq)["err"])
    errs = np.array(errs)
    cost = np.array([oracle.promote_cost(n, cfg.dq) for n in cfg.sizes])
    prev = set()
    for budget in range(0, int(cost.sum()) + 300_000, 150_000):
        sel, K = oracle.select_topk(errs, cost, budget)
        cur = set(np.nonzero(sel)[0])
        assert prev <= cur
        prev = cur
    # raising one layer's error by adding seeded noise to its weights never drops it
    sel0, K0 = oracle.select_topk(errs, cost, 600_000)
    rng = np.random.default_rng(5)
    for i in np.nonzero(sel0)[0]:
        x = oracle.from16(synth.generate(cfg, int(i)), cfg.dtype).astype(np.float32)
        x = x + (rng.standard_normal(x.size) * 0.02).astype(np.float32)
        w2 = x.astype(np.float16).view(np.uint16)
        e2 = errs.copy()
        e2[i] = oracle.layer_error(w2, cfg.dtype, cfg.dq)["err"]
        assert e2[i] > errs[i]
        sel2, _ = oracle.select_topk(e2, cost, 600_000)
        assert sel2[i] == 1


def test_predicted_k_when_the_largest_matrices_rank_first(golden_dir):
    figs = json.load(open(os.path.join(golden_dir, "pages_figures.json")))
    gib = figs["quality_setting_extra_memory_gib"]["value"]
    for cfg, expect in ((configs.S7B, {0.2: 3, 0.5: 8, 1.0: 16}),
                        (configs.S14B, {0.2: 2, 0.5: 5, 1.0: 10})):
        sizes = np.array(cfg.sizes)
        cost = np.array([oracle.promote_cost(int(n), True) for n in sizes])
        err = sizes.astype(np.float64)     # larger matrix -> larger error
        for g, k in expect.items():
            _, K = oracle.select_topk(err, cost, int(g * (1 << 30)))
            assert K == k
            # closed form: K whole FFN matrices, each costing 2n - (n/2 + n/64 + 4 n/16384)
            ffn = int(sizes.max())
            c_ffn = 2 * ffn - (ffn // 2 + ffn // 64 + 4 * (ffn // 16384))
            assert k == int(g * (1 << 30)) // c_ffn
    assert gib == 0.2


def test_toy_stack_promotes_two():
    cfg = configs.TOY
    errs = np.array([oracle.layer_error(synth.generate(cfg, i), cfg.dtype, cfg.dq)["err"]
                     for i in range(cfg.n_layers)])
    cost = np.array([oracle.promote_cost(n, cfg.dq) for n in cfg.sizes])
    sel, K = oracle.select_topk(errs, cost, -1, cfg.kcap)
    assert K == 2
    top2 = set(np.argsort(-errs, kind="stable")[:2])
    assert set(np.nonzero(sel)[0]) == top2
    # the FFN matrices hold 2.7x the elements of the attention ones
    assert all(cfg.layers[i][0].split(".")[1] in ("gate", "up", "down") for i in top2)
