"""GPU parity of the selection variants and the squared norm.

nf4_layer_error_norm: err bitwise equal to nf4_layer_error's, sumsq within
1e-5 relative of the oracle's (fp32 over each lane's 64 weights, fp64 beyond;
observed far below), on ragged sizes, zero and extreme-absmax blocks, bf16
and fp16.  aqlora_select: selected set and unit count bit-exact against the
oracle on the same scores, over score divisors x groups x budget rules, with
ties, caps, no budget, and up to 65,536 layers.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_lora_fine_nf4_amd as q
import synth
from conftest import print_case
from gpu_util import layer_error, layerset, workspace

pytestmark = pytest.mark.gpu

RTOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    q.lib()
    yield
    torch.cuda.synchronize()


def _layers(dtype):
    rng = np.random.default_rng(77 + dtype)
    L = [synth.generate_raw(900 + k, n, dtype=dtype, outlier_frac=0.003)
         for k, n in enumerate([1, 63, 64, 65, 1000, 16383, 16384, 16385, 3 * 16384 + 5, 70_001])]
    z = np.zeros(16384 + 64, np.uint16)
    L.append(z)                                            # all zero: sumsq 0
    big = synth.generate_raw(950, 64 * 256, dtype=dtype)
    x = oracle.from16(big, dtype)
    x[rng.integers(0, x.size, 30)] *= 1e3 if dtype == q.NF4_FP16 else 1e30   # huge absmax blocks
    L.append(oracle.to16_rne(x, dtype))
    if dtype == q.NF4_BF16:
        e = rng.integers(0x0A00, 0x0D00, 64 * 300).astype(np.uint16)     # absmax < 2^-100
        L.append(e)
        h = rng.integers(0x7E00, 0x7F7F, 64 * 40).astype(np.uint16)      # up to 3.4e38
        h |= (rng.integers(0, 2, h.size).astype(np.uint16) << 15)
        L.append(h)
    return L


@pytest.mark.parametrize("dq", [False, True], ids=["nodq", "dq"])
@pytest.mark.parametrize("dtype", [q.NF4_BF16, q.NF4_FP16], ids=["bf16", "fp16"])
def test_layer_error_norm(dtype, dq):
    f = q.fmt(dtype, dq)
    ws_list = _layers(dtype)
    print_case("layer_error_norm", dtype, dq, [w.size for w in ws_list])
    ls = layerset(ws_list, f)
    err1 = layer_error(ls, f)
    ws = workspace(ls.ns, f)
    err2 = torch.full_like(err1, float("nan"))
    sq = torch.full_like(err1, float("nan"))
    q.nf4_layer_error_norm(ls, f, err2, sq, ws)
    torch.cuda.synchronize()
    assert torch.equal(err1.view(torch.int64), err2.view(torch.int64)), "err differs from nf4_layer_error"
    got = sq.cpu().numpy()
    worst = 0.0
    for i, w in enumerate(ws_list):
        ref = oracle.sumsq(w, dtype)
        if ref == 0.0:
            assert got[i] == 0.0
            continue
        r = abs(got[i] - ref) / ref
        worst = max(worst, r)
        assert r <= RTOL, (i, got[i], ref)
    print(f"sumsq worst relative difference {worst:.2e}", flush=True)


def _select_case(rng, nl, grouped, with_denom, rule):
    err = rng.random(nl) ** 3 * 10
    err[rng.integers(0, nl, max(1, nl // 5))] = err[0]          # ties
    cost = rng.integers(1, 1 << 22, nl).astype(np.int64)
    denom = rng.integers(1, 1 << 30, nl).astype(np.float64) if with_denom else None
    ge = None
    if grouped:
        cuts = np.sort(rng.choice(np.arange(1, nl), size=min(nl - 1, max(0, nl // 4)),
                                  replace=False)) if nl > 1 else np.array([], np.int64)
        ge = np.r_[cuts, nl].astype(np.int32)
    total = int(cost.sum())
    budget = int(rng.choice([-1, 0, total // 7, total // 2, total + 1]))
    kcap = int(rng.choice([-1, 0, 1, max(1, nl // 3)]))
    return err, cost, denom, ge, budget, kcap


@pytest.mark.parametrize("rule", [q.AQLORA_PREFIX, q.AQLORA_FILL], ids=["prefix", "fill"])
@pytest.mark.parametrize("grouped", [False, True], ids=["layers", "groups"])
@pytest.mark.parametrize("with_denom", [False, True], ids=["sse", "divided"])
@pytest.mark.parametrize("nl", [1, 2, 9, 280, 4097, 65536])
def test_select_variants_match_oracle(nl, with_denom, grouped, rule):
    rng = np.random.default_rng(nl * 8 + 4 * with_denom + 2 * grouped + rule)
    ws = torch.empty(q.aqlora_workspace_bytes(nl), dtype=torch.uint8, device="cuda")
    reps = 6 if nl <= 4097 else 2
    for rep in range(reps):
        err, cost, denom, ge, budget, kcap = _select_case(rng, nl, grouped, with_denom, rule)
        print_case("aqlora_select", nl, "denom" if with_denom else "-", "groups" if grouped else "-",
                   rule, budget, kcap, rep)
        d_err = torch.from_numpy(err).cuda()
        d_cost = torch.from_numpy(cost).cuda()
        d_den = None if denom is None else torch.from_numpy(denom).cuda()
        sel = torch.full((nl,), 7, dtype=torch.uint8, device="cuda")
        k = torch.full((1,), -5, dtype=torch.int32, device="cuda")
        q.aqlora_select(d_err, d_cost, budget, kcap, sel, k, ws, denom=d_den, group_end=ge,
                        rule=rule)
        ref_sel, ref_k = oracle.select(err, cost, budget, kcap, denom=denom, group_end=ge,
                                       rule=rule)
        torch.cuda.synchronize()
        assert k.item() == ref_k, (k.item(), ref_k)
        assert np.array_equal(sel.cpu().numpy(), ref_sel)


def test_select_with_no_options_is_select_topk():
    rng = np.random.default_rng(5)
    nl = 3000
    err = rng.random(nl)
    cost = rng.integers(1, 1000, nl).astype(np.int64)
    d_err, d_cost = torch.from_numpy(err).cuda(), torch.from_numpy(cost).cuda()
    ws = torch.empty(q.aqlora_workspace_bytes(nl), dtype=torch.uint8, device="cuda")
    for budget in (-1, 0, 12345, 400000):
        s1 = torch.empty(nl, dtype=torch.uint8, device="cuda")
        s2 = torch.empty_like(s1)
        k1 = torch.empty(1, dtype=torch.int32, device="cuda")
        k2 = torch.empty_like(k1)
        q.aqlora_select_topk(d_err, d_cost, budget, -1, s1, k1, ws)
        q.aqlora_select(d_err, d_cost, budget, -1, s2, k2, ws)
        torch.cuda.synchronize()
        assert torch.equal(s1, s2) and k1.item() == k2.item()


def test_relative_and_block_selection_end_to_end():
    """The toy stack: relative scores from the fused pass, promoted by
    transformer block, against the oracle run on the oracle's own scores."""
    from synth import configs
    cfg = configs.BY_NAME["toy"]
    f = q.fmt(cfg.dtype, cfg.dq)
    ws_list = [synth.generate(cfg, i) for i in range(cfg.n_layers)]
    ls = layerset(ws_list, f)
    ws = workspace(ls.ns, f)
    err = torch.empty(cfg.n_layers, dtype=torch.float64, device="cuda")
    sq = torch.empty_like(err)
    q.nf4_layer_error_norm(ls, f, err, sq, ws)
    cost = np.array([q.aqlora_promote_cost(n, f) for n in cfg.sizes], np.int64)
    m = len(cfg.per_block)
    ge = np.arange(m, cfg.n_layers + 1, m, dtype=np.int32)
    sws = torch.empty(q.aqlora_workspace_bytes(cfg.n_layers), dtype=torch.uint8, device="cuda")
    sel = torch.empty(cfg.n_layers, dtype=torch.uint8, device="cuda")
    k = torch.empty(1, dtype=torch.int32, device="cuda")
    budget = int(cost[:m].sum())                        # room for one block
    q.aqlora_select(err, torch.from_numpy(cost).cuda(), budget, -1, sel, k, sws, denom=sq,
                    group_end=ge, rule=q.AQLORA_FILL)
    torch.cuda.synchronize()
    o_err = np.array([oracle.layer_error(w, cfg.dtype, cfg.dq)["err"] for w in ws_list])
    o_sq = np.array([oracle.sumsq(w, cfg.dtype) for w in ws_list])
    g_err, g_sq = err.cpu().numpy(), sq.cpu().numpy()
    assert np.all(np.abs(g_err - o_err) <= RTOL * o_err)
    assert np.all(np.abs(g_sq - o_sq) <= RTOL * o_sq)
    # parity on the GPU's own scores, then the same choice from the oracle's scores
    got = sel.cpu().numpy()
    ref_sel, ref_k = oracle.select(g_err, cost, budget, -1, denom=g_sq, group_end=ge, rule=1)
    assert k.item() == ref_k == 1
    assert np.array_equal(got, ref_sel)
    o_sel, o_k = oracle.select(o_err, cost, budget, -1, denom=o_sq, group_end=ge, rule=1)
    scores = np.add.reduceat(o_err / o_sq, np.r_[0, ge[:-1]])
    gap = abs(scores[0] - scores[1]) / max(scores)
    print(f"block scores {scores}, relative gap {gap:.2e}", flush=True)
    assert gap > 1e-6 and o_k == 1 and np.array_equal(got, o_sel)
