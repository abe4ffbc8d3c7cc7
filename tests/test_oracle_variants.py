"""Pins for the oracle's selection variants and squared norm (CPU only).

The pages name the score (NF4 reconstruction error), a memory budget, top-K
and a speed setting that adapts only the top blocks (AQLoRA listing, English
abstract; aitrending page, Technical Details); the variants are readings of
those words, so they are pinned by brute force and by invariants rather than
by printed values:
  * the fill rule's choice is the lexicographically greatest feasible set in
    rank order when costs are non-negative (feasibility -- cost within budget,
    count within the cap -- is then closed under taking subsets, so greedy is
    exactly that maximum; promotion costs are always positive);
  * the prefix rule's choice is the longest feasible prefix of the ranking;
  * fill contains prefix; equal costs make them agree; singleton groups equal
    single layers; groups equal single layers over pre-summed arrays;
  * score divisors: a common power-of-two factor changes nothing;
  * sum of squares equals the exact rational sum.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle

BF16, FP16 = oracle.BF16, oracle.FP16


def _rank(scores):
    return sorted(range(len(scores)), key=lambda u: (-scores[u], u))


def _brute(scores, costs, budget, kcap):
    """-> (prefix set, fill set) by enumeration, as sets of unit indices."""
    order = _rank(scores)
    nu = len(scores)

    def feasible(S):
        return (kcap < 0 or len(S) <= kcap) and (budget < 0 or sum(costs[u] for u in S) <= budget)

    k = 0
    while k < nu and feasible(order[:k + 1]):
        k += 1
    prefix = set(order[:k])
    best = None
    for bits in itertools.product((1, 0), repeat=nu):   # lexicographic, greatest first
        S = [order[r] for r in range(nu) if bits[r]]
        if feasible(S):
            best = set(S)
            break
    return prefix, best


def _units(sel, group_end=None):
    if group_end is None:
        return {i for i in range(sel.size) if sel[i]}
    taken, b = set(), 0
    for g, e in enumerate(group_end):
        vals = set(sel[b:e].tolist())
        assert len(vals) == 1, "a group is promoted whole or not at all"
        if sel[b]:
            taken.add(g)
        b = e
    return taken


@pytest.mark.parametrize("seed", range(60))
def test_rules_equal_brute_force(seed):
    rng = np.random.default_rng(seed)
    nu = int(rng.integers(1, 10))
    scores = rng.integers(0, 5, nu).astype(np.float64)          # many ties
    costs = rng.integers(-2, 9, nu).astype(np.int64)             # negative costs allowed
    budget = int(rng.integers(-1, 20))
    kcap = int(rng.integers(-1, nu + 1))
    prefix, _ = _brute(scores.tolist(), costs.tolist(), budget, kcap)
    sp, kp = oracle.select(scores, costs, budget, kcap, rule=oracle.PREFIX)
    assert _units(sp) == prefix and kp == len(prefix)
    costs = np.abs(costs)
    _, fill = _brute(scores.tolist(), costs.tolist(), budget, kcap)
    sf, kf = oracle.select(scores, costs, budget, kcap, rule=oracle.FILL)
    assert _units(sf) == fill and kf == len(fill)


@pytest.mark.parametrize("seed", range(40))
def test_prefix_rule_is_the_topk_rule(seed):
    rng = np.random.default_rng(100 + seed)
    nl = int(rng.integers(1, 300))
    err = rng.standard_normal(nl) ** 2
    err[rng.integers(0, nl, nl // 4)] = err[0]                   # ties
    cost = rng.integers(0, 1 << 20, nl)
    budget = int(rng.integers(-1, 1 << 24))
    kcap = int(rng.integers(-1, nl + 2))
    s1, k1 = oracle.select(err, cost, budget, kcap)
    s2, k2 = oracle.select_topk(err, cost, budget, kcap)
    assert k1 == k2 and np.array_equal(s1, s2)


@pytest.mark.parametrize("seed", range(30))
def test_fill_contains_prefix_and_is_maximal(seed):
    rng = np.random.default_rng(200 + seed)
    nl = int(rng.integers(1, 200))
    err = rng.random(nl)
    cost = rng.integers(1, 1000, nl)
    budget = int(rng.integers(0, 50000))
    sp, _ = oracle.select(err, cost, budget, -1, rule=oracle.PREFIX)
    sf, kf = oracle.select(err, cost, budget, -1, rule=oracle.FILL)
    assert np.all(sf >= sp)
    used = int(cost[sf == 1].sum())
    assert used <= budget
    assert np.all(cost[sf == 0] > budget - used)                 # nothing left that fits
    assert kf == int(sf.sum())


def test_equal_costs_make_the_rules_agree():
    rng = np.random.default_rng(7)
    for _ in range(50):
        nl = int(rng.integers(1, 100))
        err = rng.random(nl)
        cost = np.full(nl, int(rng.integers(1, 100)))
        budget = int(rng.integers(0, 5000))
        assert np.array_equal(oracle.select(err, cost, budget, rule=0)[0],
                              oracle.select(err, cost, budget, rule=1)[0])


def test_budget_above_total_takes_everything_up_to_the_cap():
    err = np.linspace(1, 2, 20)
    cost = np.arange(20) + 1
    for rule in (0, 1):
        sel, k = oracle.select(err, cost, int(cost.sum()), -1, rule=rule)
        assert k == 20 and sel.all()
        sel, k = oracle.select(err, cost, int(cost.sum()), 5, rule=rule)
        assert k == 5 and set(np.flatnonzero(sel)) == set(range(15, 20))


@pytest.mark.parametrize("rule", [0, 1])
def test_singleton_groups_equal_single_layers(rule):
    rng = np.random.default_rng(11)
    for _ in range(40):
        nl = int(rng.integers(1, 120))
        err = rng.random(nl)
        cost = rng.integers(0, 100, nl)
        budget, kcap = int(rng.integers(-1, 3000)), int(rng.integers(-1, nl))
        a = oracle.select(err, cost, budget, kcap, rule=rule)
        b = oracle.select(err, cost, budget, kcap, rule=rule, group_end=np.arange(1, nl + 1))
        assert a[1] == b[1] and np.array_equal(a[0], b[0])


@pytest.mark.parametrize("rule", [0, 1])
def test_groups_equal_single_layers_over_summed_arrays(rule):
    """Integer-valued scores make every group sum exact, so ranking groups is
    ranking their pre-summed scores."""
    rng = np.random.default_rng(12)
    for _ in range(40):
        ng = int(rng.integers(1, 40))
        sizes = rng.integers(1, 8, ng)
        ge = np.cumsum(sizes).astype(np.int32)
        nl = int(ge[-1])
        err = rng.integers(0, 50, nl).astype(np.float64)
        cost = rng.integers(0, 100, nl)
        gs = np.add.reduceat(err, np.r_[0, ge[:-1]])
        gc = np.add.reduceat(cost, np.r_[0, ge[:-1]])
        budget, kcap = int(rng.integers(-1, 4000)), int(rng.integers(-1, ng))
        sg, kg = oracle.select(err, cost, budget, kcap, rule=rule, group_end=ge)
        su, ku = oracle.select(gs, gc, budget, kcap, rule=rule)
        assert kg == ku
        assert np.array_equal(sg, np.repeat(su, sizes))


def test_score_divisors():
    rng = np.random.default_rng(13)
    for _ in range(40):
        nl = int(rng.integers(1, 150))
        err = rng.random(nl) * 1e3
        cost = rng.integers(0, 100, nl)
        n = rng.integers(1, 1 << 20, nl).astype(np.float64)
        budget = int(rng.integers(0, 5000))
        base = oracle.select(err, cost, budget, denom=n)
        scaled = oracle.select(err, cost, budget, denom=n * 2.0 ** int(rng.integers(-40, 40)))
        assert np.array_equal(base[0], scaled[0])
        # a common divisor changes nothing; 1 is the identity
        assert np.array_equal(oracle.select(err, cost, budget, denom=np.full(nl, 3.0))[0],
                              oracle.select(err, cost, budget)[0])
        assert np.array_equal(oracle.select(err, cost, budget, denom=np.ones(nl))[0],
                              oracle.select(err, cost, budget)[0])
    # the divisor reorders: equal errors, different sizes -> smaller matrix first
    sel, k = oracle.select([5.0, 5.0], [1, 1], 1, denom=[100.0, 10.0])
    assert k == 1 and sel.tolist() == [0, 1]


def _bits_to_fraction(h, dtype):
    v = oracle.from16(np.array([h], np.uint16), dtype)[0]
    return Fraction(float(v))


@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_sumsq_is_the_exact_sum(dtype):
    rng = np.random.default_rng(14 + dtype)
    for _ in range(30):
        n = int(rng.integers(1, 400))
        w = rng.integers(0, 1 << 16, n).astype(np.uint16)
        # keep finite values only
        e = (w >> 7) & 0xFF if dtype == BF16 else (w >> 10) & 0x1F
        w[e == (0xFF if dtype == BF16 else 0x1F)] &= 0x8000
        exact = sum(_bits_to_fraction(int(h), dtype) ** 2 for h in w)
        got = oracle.sumsq(w, dtype)
        assert got == float(exact) or abs(Fraction(got) - exact) <= exact * Fraction(1, 1 << 52)


def test_sumsq_closed_forms():
    one = np.full(1000, 0x3F80, np.uint16)          # bf16 1.0
    assert oracle.sumsq(one, BF16) == 1000.0
    half = np.full(64, 0xBF00, np.uint16)           # bf16 -0.5
    assert oracle.sumsq(half, BF16) == 16.0
    assert oracle.sumsq(np.zeros(17, np.uint16), BF16) == 0.0
    assert oracle.sumsq(np.array([0x3C00, 0x4000], np.uint16), FP16) == 5.0   # fp16 1, 2
