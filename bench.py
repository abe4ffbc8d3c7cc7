"""Benchmark: GB/s of 16-bit weights through the NF4 codec and the AQLoRA pass.

One step over the 14B-shaped synthetic stack (40 blocks x 7 matrices, d=5120,
ffn=13824, bf16 N(0,0.02) with 0.05% x10 outliers, 12.69 G weights):
  1. nf4_layer_error   -- fused absmax / NF4 encode / int8 double quant /
                          in-register dequant / squared error, all 280 matrices
  2. aqlora_select_topk -- rank by error, promote the top-K under 0.2 GiB
  3. nf4_dequantize x2  -- every matrix left in NF4 back to bf16, twice (one
                          training step's forward + backward dequant traffic)
value = 16-bit weight bytes through the codec per second: the fused pass reads
2 bytes per weight, each dequant pass writes 2 bytes per unpromoted weight.

Prints one JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GB/s of bf16 weights through NF4 quant+dequant+error; % of HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, 8 TB/s
# VALU issue peak: 256 CUs x 4 SIMDs, one wave64 vector instruction per SIMD every
# 4 cycles (16 lanes wide) at 2.4 GHz = 614.4 G wave-instructions/s
VALU_PEAK_GIPS = 256 * 4 * 2.4 / 4
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_bytes_per_weight(dq: bool) -> float:
    """Bytes each kernel must move per weight: 16-bit weight once, half a byte
    of code, and the constants (int8 per 64 + fp32 per 16384, or fp32 per 64)."""
    return 2.0 + 0.5 + ((1.0 / 64 + 4.0 / 16384) if dq else 4.0 / 64)


# the files that define the fused codec and dequantisation kernels and their launches
CODEC_SOURCES = ("k_codec.hip", "nf4_format.h", "nf4_internal.h")


def source_hash(names=None) -> str:
    """Hash of the kernel sources (all of them, or the named ones)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_lora_fine_nf4_amd", "csrc")
    for name in sorted(names if names is not None else os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def codec_source_hash() -> str:
    return source_hash(CODEC_SOURCES)


def read_profile_value(name: str, key: str):
    """A value from a committed counter summary (`key=value` lines), if the
    summary was taken on the current sources of the codec kernels (else None)."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#") and not line.startswith(" "):
            k, v = line.strip().split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("codec_source_hash") != codec_source_hash():
        return None
    v = vals.get(key)
    return float(v) if v else None


def read_traffic(workload_key: str, kernel: str):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary."""
    return read_profile_value(f"traffic_{workload_key}.txt", f"{kernel}_bytes_per_launch")


def alu_roofline(workload_key: str, kernel: str, weights: int, ms: float):
    """The kernel against the VALU issue peak: vector instructions per weight
    from the committed SQ_INSTS_VALU summary (same sources only), times the
    weights of one launch, over the launch time measured here."""
    vpw = read_profile_value(f"counters_{workload_key}.txt", f"{kernel}_valu_per_weight")
    if vpw is None:
        return None
    gips = vpw * weights / 64 / (ms * 1e-3) / 1e9
    return {"bound": "alu", "valu_per_weight": vpw, "achieved": round(gips, 1),
            "peak": VALU_PEAK_GIPS, "unit": "G wave64 VALU instructions/s",
            "frac": round(gips / VALU_PEAK_GIPS, 4)}


def cpu_pass(cfg, n_total: int, blocks: int = 1):
    """The multi-threaded host-CPU scoring pass (libnf4cpu.so, not the oracle)
    on the first transformer block(s) of the stack, all host threads and one,
    with the full-stack time it implies (the pass streams, so its rate does
    not depend on the size)."""
    import quantized_lora_fine_nf4_amd as q
    from quantized_lora_fine_nf4_amd import cpu
    import synth
    f = q.fmt(cfg.dtype, cfg.dq)
    m = len(cfg.per_block)
    idx = list(range(min(cfg.n_layers, blocks * m)))
    ws = [synth.generate(cfg, i) for i in idx]
    n = sum(w.size for w in ws)
    res = {"sample": f"first {len(idx)} matrices ({n} weights) of the stack", "weights": n}
    for name, th in (("all_threads", 0), ("one_thread", 1)):
        cpu.layer_error(ws, f, threads=th, with_absmax=not cfg.dq)   # warm (first touch)
        t0 = time.perf_counter()
        cpu.layer_error(ws, f, threads=th, with_absmax=not cfg.dq)
        dt = time.perf_counter() - t0
        res[name] = {"GBps": round(2.0 * n / dt / 1e9, 3), "s": round(dt, 3),
                     "threads": cpu.max_threads() if th == 0 else 1,
                     "full_stack_s": round(dt * n_total / n, 2)}
    return res


def cpu_baseline(cfg, seconds: float, n_deq: int, n_total: int):
    """The oracle (single-threaded C), untuned, on a bounded sample of the same
    workload: slices of 64 double-quant groups from successive matrices."""
    import numpy as np
    import oracle
    import synth
    slice_n = 64 * 16384
    done, t_fused, t_deq = 0, 0.0, 0.0
    i = 0
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})         # the timed work on one core
    try:
        while t_fused + t_deq < seconds:
            w = synth.generate(cfg, i % cfg.n_layers, first=0,
                               count=min(slice_n, cfg.n(i % cfg.n_layers)), threads=1)
            t0 = time.perf_counter()
            r = oracle.layer_error(w, cfg.dtype, cfg.dq)
            t1 = time.perf_counter()
            consts = (dict(qabsmax=r["qabsmax"], scale2=r["scale2"]) if cfg.dq
                      else dict(absmax=r["absmax"]))
            y = oracle.dequantize(r["codes"], w.size, cfg.dtype, **consts)
            t2 = time.perf_counter()
            assert np.array_equal(y, r["y"])
            t_fused += t1 - t0
            t_deq += t2 - t1
            done += w.size
            i += 1
    finally:
        os.sched_setaffinity(0, allowed)
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    per_w_fused = t_fused / done
    per_w_deq = t_deq / done
    step_s = per_w_fused * n_total + cfg.dequant_repeats * per_w_deq * n_deq
    weight_bytes = 2.0 * n_total + cfg.dequant_repeats * 2.0 * n_deq
    return {
        "value": weight_bytes / step_s / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "cpu": {"model": model, "pinned_core": core, "cores_available": len(allowed),
                "compiler": " ".join(oracle.BUILD_FLAGS)},
        "sample": (f"{done} weights ({i} slices of 64 double-quant groups, first slice of "
                   f"successive matrices): fused oracle pass {t_fused:.2f} s "
                   f"({2 * done / t_fused / 1e6:.1f} MB/s of bf16), oracle dequant "
                   f"{t_deq:.2f} s; scaled to one full step"),
    }


def hbm_probe(torch):
    """Achievable HBM streaming rates on this device with PyTorch's own kernels
    over 8 GiB buffers (far beyond the 256 MB last-level cache): write-only
    (fill), read+write (copy) and read-only (the fastest of a few reductions)."""
    nbytes = 8 << 30
    a = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(7)
    res = {}

    def rate(fn, moved, reps=6):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(moved / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)

    res["write_GBps"] = rate(lambda: b.fill_(3), nbytes)
    res["copy_GBps"] = rate(lambda: b.copy_(a), 2 * nbytes)
    reads = {
        "amax_i32": lambda: a.amax(),
        "amax_i64": lambda: a.view(torch.int64).amax(),
        "sum_f32": lambda: a.view(torch.float32).sum(),
        "count_nonzero_i64": lambda: torch.count_nonzero(a.view(torch.int64)),
    }
    read_rates = {k: rate(fn, nbytes) for k, fn in reads.items()}
    best = max(read_rates, key=read_rates.get)
    res["read_GBps"] = read_rates[best]
    res["read_op"] = best
    res["read_candidates_GBps"] = read_rates
    res["buffer_bytes"] = nbytes
    return res


def selections(q, torch, err, cost, cfg, stream, reps=20):
    """aqlora_select_topk at every budget of the configuration, on the GPU's
    scores of the last step: K, the relative score gap at the cut, and the
    call's time (launches included)."""
    import numpy as np
    nl = int(err.numel())
    sws = torch.empty(q.aqlora_workspace_bytes(nl), dtype=torch.uint8, device="cuda")
    sel = torch.empty(nl, dtype=torch.uint8, device="cuda")
    k = torch.empty(1, dtype=torch.int32, device="cuda")
    errs = err.cpu().numpy()
    order = np.lexsort((np.arange(nl), -errs))
    res = {}
    for g, b in zip(cfg.budgets_gib, cfg.budgets_bytes()):
        q.aqlora_select_topk(err, cost, b, cfg.kcap, sel, k, sws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            q.aqlora_select_topk(err, cost, b, cfg.kcap, sel, k, sws)
        e1.record(stream)
        torch.cuda.synchronize()
        K = int(k.item())
        gap = None
        if 0 < K < nl:
            a, c = errs[order[K - 1]], errs[order[K]]
            gap = float((a - c) / a)
        res[f"{g} GiB"] = {"budget_bytes": b, "K": K, "relative_gap_at_cut": gap,
                           "select_us": round(e0.elapsed_time(e1) / reps * 1e3, 1)}
    return res


def variants(q, torch, ls, f, err, cost, budget, cfg, stream, ws, fused_bytes, reps=10):
    """Selection variants on the same stack, after the timed steps: the fused
    pass that also returns the sum of squares (relative scores), and the
    selector with relative scores, transformer-block units and both budget
    rules.  Mean launch time from events on the launch stream."""
    nl = cfg.n_layers

    def timed(fn):
        fn()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for r in range(reps):
            e[2 * r].record(stream)
            fn()
            e[2 * r + 1].record(stream)
        torch.cuda.synchronize()
        return sum(e[2 * r].elapsed_time(e[2 * r + 1]) for r in range(reps)) / reps

    sq = torch.empty_like(err)
    res = {}
    t_plain = timed(lambda: q.nf4_layer_error(ls, f, err, ws))
    t_norm = timed(lambda: q.nf4_layer_error_norm(ls, f, err, sq, ws))
    res["nf4_layer_error_ms"] = round(t_plain, 4)
    res["nf4_layer_error_norm_ms"] = round(t_norm, 4)
    e, q2 = err.cpu().double(), sq.cpu().double()
    n = torch.tensor([float(x) for x in cfg.sizes], dtype=torch.float64)
    rel = e / q2
    res["error_stats"] = {   # the GPU pass's own scores: SSE, MSE = SSE / n, relative = SSE / sum x^2
        "sse_total": float(e.sum()), "mse_mean": float((e / n).mean()),
        "relative_mean": float(rel.mean()), "relative_min": float(rel.min()),
        "relative_max": float(rel.max())}
    res["nf4_layer_error_norm_GBps"] = round(fused_bytes / (t_norm * 1e-3) / 1e9, 1)
    # the standalone calls of the boundary on the whole stack: nf4_quantize
    # (absmax, codes and, with double quant, the second level; no error) on a
    # set that shares the stack's weights and codes and adds the fp32 absmax it
    # writes, then nf4_double_quant of those absmax values
    qs = q.LayerSet(cfg.sizes, f, with_absmax=True, with_out=False, w=ls.w, codes=ls.codes)
    qws = torch.empty(q.nf4_workspace_bytes(qs.ns, f), dtype=torch.uint8, device="cuda")
    n_all = cfg.total
    ngroups = sum((n + 16383) // 16384 for n in cfg.sizes)
    t_q = timed(lambda: q.nf4_quantize(qs, f, qws))
    qb = 2.5 * n_all + 4.0 * n_all / 64 + ((n_all / 64 + 4.0 * ngroups) if cfg.dq else 0.0)
    res["nf4_quantize_ms"] = round(t_q, 4)
    res["nf4_quantize_GBps"] = round(qb / (t_q * 1e-3) / 1e9, 1)
    res["nf4_quantize_frac_of_peak"] = round(qb / (t_q * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    if cfg.dq:
        t_dq = timed(lambda: q.nf4_double_quant(qs, f, qws))
        db = 4.0 * n_all / 64 + n_all / 64 + 4.0 * ngroups   # absmax read, int8 and scale2 written
        res["nf4_double_quant_ms"] = round(t_dq, 4)
        res["nf4_double_quant_GBps"] = round(db / (t_dq * 1e-3) / 1e9, 1)
        res["nf4_double_quant_frac_of_peak"] = round(db / (t_dq * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    del qs, qws
    m = len(cfg.per_block)
    ge = list(range(m, nl + 1, m))
    sws = torch.empty(q.aqlora_workspace_bytes(nl), dtype=torch.uint8, device="cuda")
    sel = torch.empty(nl, dtype=torch.uint8, device="cuda")
    k = torch.empty(1, dtype=torch.int32, device="cuda")
    sel_us = {}
    for name, kw in (("topk", None),
                     ("relative_prefix", dict(denom=sq)),
                     ("relative_fill", dict(denom=sq, rule=q.AQLORA_FILL)),
                     ("blocks_prefix", dict(group_end=ge)),
                     ("relative_blocks_fill", dict(denom=sq, group_end=ge, rule=q.AQLORA_FILL))):
        if kw is None:
            fn = lambda: q.aqlora_select_topk(err, cost, budget, cfg.kcap, sel, k, sws)
        else:
            fn = lambda kw=kw: q.aqlora_select(err, cost, budget, cfg.kcap, sel, k, sws, **kw)
        sel_us[name] = round(timed(fn) * 1e3, 1)
    res["select_us"] = sel_us
    res["select_layers"] = nl
    return res


def codec_variants(q, torch, ls, cfg, stream, reps=5):
    """The codec at block sizes 32-256 with each second-level kind on the
    whole stack: the error pass (absmax, mean, second level, codes, error)
    and the dequantisation.  Weights, codes and outputs are the stack's own
    buffers; only the constants are allocated per block size.  GB/s count
    the bytes the format must move per weight (16-bit weight, half a byte
    of code, the stored constants), though the error pass reads the weights
    twice (the mean of the kinds with an offset needs every absmax first)."""
    nl = cfg.n_layers
    n_total = cfg.total
    err = torch.empty(nl, dtype=torch.float64, device="cuda")
    mean = torch.empty(nl, dtype=torch.float32, device="cuda")

    def timed(fn):
        fn()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for r in range(reps):
            e[2 * r].record(stream)
            fn()
            e[2 * r + 1].record(stream)
        torch.cuda.synchronize()
        return sum(e[2 * r].elapsed_time(e[2 * r + 1]) for r in range(reps)) / reps

    kinds = (("none", q.NF4_DQ_NONE), ("int8", q.NF4_DQ_INT8),
             ("int8_mean", q.NF4_DQ_INT8_MEAN), ("e4m3_mean", q.NF4_DQ_E4M3_MEAN))
    res = {}
    for block in (32, 64, 128, 256):
        vs = q.LayerSet(cfg.sizes, q.fmt(cfg.dtype, True), with_absmax=True, w=ls.w,
                        codes=ls.codes, out=ls.out, block=block)
        ws = torch.empty(q.nf4_workspace_bytes_variant(vs.ns, q.variant(cfg.dtype, block, 0)),
                         dtype=torch.uint8, device="cuda")
        for kname, kind in kinds:
            v = q.variant(cfg.dtype, block, kind)
            store = sum(q.nf4_storage_bytes_variant(n, v) for n in cfg.sizes)
            t_e = timed(lambda: q.nf4_layer_error_variant(vs, v, err, ws, mean=mean))
            t_d = timed(lambda: q.nf4_dequantize_variant(vs, v, ws, mean=mean))
            moved = 2.0 * n_total + store
            res[f"b{block}_{kname}"] = {
                "error_ms": round(t_e, 3), "error_GBps": round(moved / (t_e * 1e-3) / 1e9, 1),
                "dequant_ms": round(t_d, 3), "dequant_GBps": round(moved / (t_d * 1e-3) / 1e9, 1),
                "bits_per_weight": round(8.0 * store / n_total, 4)}
        del vs, ws
    return res


MFMA_BF16_PEAK_TFS = 2500.0


def matmul_block(q, torch, ls, f, cfg, stream, deq_ms_per_weight, keep, m=4096, reps=10):
    """The NF4 weight consumed by its matmul (fused dequantisation on the
    matrix cores) on one FFN up-projection of the stack, m tokens, against
    the library bf16 GEMM on the dequantised weight plus a standalone
    dequantisation of it (the dequantise-then-multiply pattern).  The
    dequantisation time is the stack's measured per-weight rate times this
    matrix's size (a separate small launch would mix into the per-kernel
    profile of the full-stack launches)."""
    names = [nm for nm, _, _ in cfg.per_block]
    pos = names.index("up") if "up" in names else 0
    # the first such matrix that the step dequantised (a promoted one has no 16-bit copy here)
    li = next(b * len(names) + pos for b in range(cfg.blocks) if b * len(names) + pos in keep)
    _, rows, cols = cfg.per_block[pos]
    layer = ls.c_layers[li]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    x = torch.randn(m, cols, dtype=torch.bfloat16, device="cuda", generator=gen)
    gy = torch.randn(m, rows, dtype=torch.bfloat16, device="cuda", generator=gen)
    yf = torch.empty(m, rows, dtype=torch.bfloat16, device="cuda")
    yb = torch.empty(m, cols, dtype=torch.bfloat16, device="cuda")

    def timed_once(fn):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for r in range(reps):
            e[2 * r].record(stream)
            fn()
            e[2 * r + 1].record(stream)
        torch.cuda.synchronize()
        return sum(e[2 * r].elapsed_time(e[2 * r + 1]) for r in range(reps)) / reps

    def timed_arms(arms, rounds=5, warm_ms=1000.0):
        """Mean launch time of each arm: after two untimed calls of each (the
        library's first calls set up its kernels), the arms are run in turn
        for about warm_ms (the GPU's clock settles only after a sustained
        load: the library GEMM here runs ~15% faster after a second of work
        than in its first tens of milliseconds), then timed in alternating
        rounds; each arm's median round is kept, so that no arm is timed in a
        different clock state than the others."""
        for fn in arms:
            fn()
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < warm_ms:
            for fn in arms:
                for _ in range(5):
                    fn()
            torch.cuda.synchronize()
        res = [[] for _ in arms]
        for _ in range(rounds):
            for i, fn in enumerate(arms):
                res[i].append(timed_once(fn))
        return [sorted(r)[len(r) // 2] for r in res]

    t_deq = deq_ms_per_weight * rows * cols
    w = ls.out_of(li).view(torch.bfloat16).view(rows, cols)   # written by the step's dequant
    wt = w.t().contiguous()
    # nf4_matmul_ws: with a workspace the tiles left over after the whole
    # rounds split their reduction instead of running as row pieces
    nwf = q.nf4_matmul_workspace_bytes(rows, cols, False, m)
    nwb = q.nf4_matmul_workspace_bytes(rows, cols, True, m)
    wsf = torch.empty(max(nwf, 1), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(max(nwb, 1), dtype=torch.uint8, device="cuda")
    t_fwd, t_bwd, t_wf, t_wb, t_lib_f, t_lib_b = timed_arms([
        lambda: q.nf4_matmul(layer, rows, cols, f, x.view(torch.int16), yf),
        lambda: q.nf4_matmul(layer, rows, cols, f, gy.view(torch.int16), yb, backward=True),
        lambda: q.nf4_matmul_ws(layer, rows, cols, f, x.view(torch.int16), yf, wsf),
        lambda: q.nf4_matmul_ws(layer, rows, cols, f, gy.view(torch.int16), yb, wsb, backward=True),
        lambda: torch.matmul(x, wt),
        lambda: torch.matmul(gy, w)])
    flops = 2.0 * m * rows * cols
    tf = lambda t: round(flops / (t * 1e-3) / 1e12, 1)
    res = {
        "shape": {"m": m, "rows": rows, "cols": cols, "matrix": f"{names[pos]} of block {li // len(names)}"},
        "fused_fwd_ms": round(t_fwd, 4), "fused_fwd_TFLOPs": tf(t_fwd),
        "fused_bwd_ms": round(t_bwd, 4), "fused_bwd_TFLOPs": tf(t_bwd),
        "library_bf16_fwd_ms": round(t_lib_f, 4), "library_bf16_fwd_TFLOPs": tf(t_lib_f),
        "library_bf16_bwd_ms": round(t_lib_b, 4), "library_bf16_bwd_TFLOPs": tf(t_lib_b),
        "dequant_ms_scaled": round(t_deq, 4),
        "dequant_then_library_fwd_ms": round(t_deq + t_lib_f, 4),
        "dequant_then_library_bwd_ms": round(t_deq + t_lib_b, 4),
        "fused_over_dequant_library_fwd": round(t_fwd / (t_deq + t_lib_f), 4),
        "fused_over_dequant_library_bwd": round(t_bwd / (t_deq + t_lib_b), 4),
        "fused_ws_fwd_ms": round(t_wf, 4), "fused_ws_fwd_TFLOPs": tf(t_wf), "fused_ws_fwd_bytes": nwf,
        "fused_ws_bwd_ms": round(t_wb, 4), "fused_ws_bwd_TFLOPs": tf(t_wb), "fused_ws_bwd_bytes": nwb,
        "fused_ws_over_dequant_library_fwd": round(t_wf / (t_deq + t_lib_f), 4),
        "fused_ws_over_dequant_library_bwd": round(t_wb / (t_deq + t_lib_b), 4),
        "roofline": {"bound": "mfma", "kernel": "nf4_matmul forward",
                     "achieved": tf(t_fwd), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(tf(t_fwd) / MFMA_BF16_PEAK_TFS, 4)},
        "roofline_bwd": {"bound": "mfma", "kernel": "nf4_matmul backward",
                         "achieved": tf(t_bwd), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": round(tf(t_bwd) / MFMA_BF16_PEAK_TFS, 4)},
    }
    # few tokens to mid m (nf4_matmul_ws: the few-token forward kernel at
    # m <= 32, the split 128 x 128 reduction at m = 128, the 256 x 256
    # kernels with a split reduction at m = 512) against dequantise + library
    # GEMM
    small = {}
    for ms in (16, 32, 128, 512):
        xs = torch.randn(ms, cols, dtype=torch.bfloat16, device="cuda", generator=gen)
        gs = torch.randn(ms, rows, dtype=torch.bfloat16, device="cuda", generator=gen)
        ysf = torch.empty(ms, rows, dtype=torch.bfloat16, device="cuda")
        ysb = torch.empty(ms, cols, dtype=torch.bfloat16, device="cuda")
        nf = q.nf4_matmul_workspace_bytes(rows, cols, False, ms)
        nb = q.nf4_matmul_workspace_bytes(rows, cols, True, ms)
        wsf = torch.empty(max(nf, 1), dtype=torch.uint8, device="cuda") if nf else None
        wsb = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda") if nb else None
        tf_, tb_, lf, lb = timed_arms([
            lambda: q.nf4_matmul_ws(layer, rows, cols, f, xs.view(torch.int16), ysf, wsf),
            lambda: q.nf4_matmul_ws(layer, rows, cols, f, gs.view(torch.int16), ysb, wsb, backward=True),
            lambda: torch.matmul(xs, wt),
            lambda: torch.matmul(gs, w)], warm_ms=200.0)
        # algorithmic bytes of the forward call: codes, int8 constants, scale2, x, out
        fbytes = rows * cols // 2 + rows * cols // 64 + rows * cols // 64 // 256 * 4 + 2 * ms * (cols + rows)
        small[f"m{ms}"] = {"fused_ws_fwd_ms": round(tf_, 4), "fused_ws_bwd_ms": round(tb_, 4),
                           "fused_ws_fwd_GBps": round(fbytes / (tf_ * 1e-3) / 1e9, 1),
                           "fused_ws_fwd_frac_of_hbm_peak": round(fbytes / (tf_ * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "library_only_fwd_ms": round(lf, 4), "library_only_bwd_ms": round(lb, 4),
                           "dequant_then_library_fwd_ms": round(t_deq + lf, 4),
                           "dequant_then_library_bwd_ms": round(t_deq + lb, 4)}
        del xs, gs, ysf, ysb, wsf, wsb
    res["small_m"] = small
    del x, gy, yf, yb, wt
    return res


def protocol_arms(launch, seconds: float, torch, stream):
    """Fixed-duration timing with a duplicated arm: the same launch is timed as
    arms A and A2 in alternating blocks of about 0.2 s until each has run for
    `seconds`; returns per-arm launch durations and their relative spread."""
    block = 1
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # size the block to ~0.2 s
    e0.record(stream)
    launch()
    e1.record(stream)
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    block = max(1, int(200.0 / one))
    tot = {"A": [0.0, 0], "A2": [0.0, 0]}
    while min(v[0] for v in tot.values()) < seconds * 1e3:
        for arm in ("A", "A2"):
            e0.record(stream)
            for _ in range(block):
                launch()
            e1.record(stream)
            torch.cuda.synchronize()
            tot[arm][0] += e0.elapsed_time(e1)
            tot[arm][1] += block
    ms = {k: v[0] / v[1] for k, v in tot.items()}
    mean = 0.5 * (ms["A"] + ms["A2"])
    return {"ms_A": round(ms["A"], 4), "ms_A2": round(ms["A2"], 4),
            "launches_each": tot["A"][1], "noise_floor_rel": round(abs(ms["A"] - ms["A2"]) / mean, 5)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="14b", help="toy | single | 1.4b | 7b | 14b")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--warm-seconds", type=float, default=0.0,
                    help="after the W warmup steps, keep stepping untimed for this long (the clock "
                         "settles only under sustained load; matters for the small stacks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip timing the selection variants, the fused matmul and the codec variants")
    ap.add_argument("--matmul", action="store_true",
                    help="time the fused matmul even with --no-variants")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="only measure achievable streaming bandwidth with PyTorch's own kernels")
    ap.add_argument("--protocol", type=float, default=0.0, metavar="SECONDS",
                    help="also time each kernel for a fixed duration as two interleaved, "
                         "identical arms (noise floor = their spread)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); "
              f"got --gpus {args.gpus}", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_lora_fine_nf4_amd as q
    import synth
    from synth import configs

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        nbytes = 1 << 31
        src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": nbytes, "launches": 3}), flush=True)
        return

    if args.hbm_probe:
        print(json.dumps(hbm_probe(torch)), flush=True)
        return

    q.lib()
    cfg = configs.BY_NAME[args.config]
    f = q.fmt(cfg.dtype, cfg.dq)
    nl = cfg.n_layers
    n_total = cfg.total
    log(f"config {cfg.name}: {nl} matrices, {n_total} weights")

    ls = q.LayerSet(cfg.sizes, f, with_absmax=not cfg.dq)
    t0 = time.time()
    synth.fill_device(cfg, [ls.w_of(i) for i in range(nl)],
                      progress=lambda i: (i % 40 == 39) and log(f"generated {i + 1}/{nl} matrices"))
    log(f"generated and uploaded in {time.time() - t0:.1f} s")

    ws = torch.empty(q.nf4_workspace_bytes(ls.ns, f), dtype=torch.uint8, device="cuda")
    err = torch.empty(nl, dtype=torch.float64, device="cuda")
    cost = torch.tensor([q.aqlora_promote_cost(n, f) for n in cfg.sizes], dtype=torch.int64,
                        device="cuda")
    sel = torch.empty(nl, dtype=torch.uint8, device="cuda")
    kout = torch.empty(1, dtype=torch.int32, device="cuda")
    sws = torch.empty(q.aqlora_workspace_bytes(nl), dtype=torch.uint8, device="cuda")
    budget = cfg.budgets_bytes()[0] if cfg.budgets_gib else -1
    stream = torch.cuda.current_stream()
    def step(events=None):
        if events is not None:
            events["fused"][0].record(stream)
        q.nf4_layer_error(ls, f, err, ws)
        if events is not None:
            events["fused"][1].record(stream)
        q.aqlora_select_topk(err, cost, budget, cfg.kcap, sel, kout, sws)
        # the promoted matrices skip dequantisation: the selection stays on the
        # device as the mask, no host round trip inside the step
        for r in range(cfg.dequant_repeats):
            if events is not None:
                events["dequant"][2 * r].record(stream)
            q.nf4_dequantize_masked(ls, f, sel, ws)
            if events is not None:
                events["dequant"][2 * r + 1].record(stream)

    def selected_keep():
        return tuple(i for i, s in enumerate(sel.cpu().tolist()) if not s)   # synchronises

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.warm_seconds > 0:
        # small stacks: W steps last a few ms, less than the GPU needs to reach
        # its sustained clock (a 1.4B fused pass takes 0.63 ms cold, 0.54 warm)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.warm_seconds:
            step()
            torch.cuda.synchronize()

    K = args.steps
    evs = [{"fused": [torch.cuda.Event(enable_timing=True) for _ in range(2)],
            "dequant": [torch.cuda.Event(enable_timing=True) for _ in range(2 * cfg.dequant_repeats)]}
           for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        step(evs[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    fused_ms = sum(e["fused"][0].elapsed_time(e["fused"][1]) for e in evs) / K
    deq_ms = [e["dequant"][2 * r].elapsed_time(e["dequant"][2 * r + 1])
              for e in evs for r in range(cfg.dequant_repeats)]
    deq_ms = sum(deq_ms) / max(1, len(deq_ms))

    keep = selected_keep()   # the same every step (deterministic); read after the timed region
    n_deq = sum(cfg.sizes[i] for i in keep)
    bpw = algorithmic_bytes_per_weight(cfg.dq)
    fused_bytes = bpw * n_total
    deq_bytes = bpw * n_deq
    weight_bytes = 2.0 * n_total + cfg.dequant_repeats * 2.0 * n_deq
    value = weight_bytes / (ms_per_step * 1e-3) / 1e9
    alg_bytes = fused_bytes + cfg.dequant_repeats * deq_bytes
    step_frac = alg_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS

    kernels = {
        "nf4_layer_error": {"ms": round(fused_ms, 4),
                            "algorithmic_GB": round(fused_bytes / 1e9, 4),
                            "GBps": round(fused_bytes / (fused_ms * 1e-3) / 1e9, 1)},
    }
    if cfg.dequant_repeats > 0:   # configurations without the dequantisation phase time the pass only
        kernels["nf4_dequantize"] = {"ms": round(deq_ms, 4), "launches_per_step": cfg.dequant_repeats,
                                     "algorithmic_GB": round(deq_bytes / 1e9, 4),
                                     "GBps": round(deq_bytes / (deq_ms * 1e-3) / 1e9, 1)}
    for k in kernels.values():
        k["frac_of_peak"] = round(k["GBps"] / HBM_PEAK_GBS, 4)
    kernels["nf4_layer_error"]["alu"] = alu_roofline(args.config, "nf4_layer_error", n_total, fused_ms)
    if "nf4_dequantize" in kernels:
        kernels["nf4_dequantize"]["alu"] = alu_roofline(args.config, "nf4_dequantize", n_deq, deq_ms)
    for name, k in kernels.items():
        k["traffic"] = read_traffic(args.config, name)
    # dominant kernel: the larger share of the step's time
    dom = "nf4_dequantize" if cfg.dequant_repeats * deq_ms > fused_ms else "nf4_layer_error"
    dk = kernels[dom]
    traffic = read_traffic(args.config, dom)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": dk["GBps"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": dk["frac_of_peak"], "traffic": traffic}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        **({"warm_seconds": args.warm_seconds} if args.warm_seconds > 0 else {}),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "matrices": nl, "weights": n_total,
                   "weights_dtype": "bf16" if cfg.dtype == 0 else "fp16",
                   "double_quant": cfg.dq, "budget_bytes": budget,
                   "promoted": nl - len(keep), "dequantized_weights": n_deq,
                   "dequant_passes": cfg.dequant_repeats},
        "hbm_frac_of_peak_step": round(step_frac, 4),
        "roofline": roofline,
        "kernels": kernels,
        "source_hash": source_hash(),
        "codec_source_hash": codec_source_hash(),
    }
    if cfg.budgets_gib:
        out["selections"] = selections(q, torch, err, cost, cfg, stream)
    if not args.no_variants:
        out["variants"] = variants(q, torch, ls, f, err, cost, budget, cfg, stream, ws, fused_bytes)
    if (not args.no_variants or args.matmul) and cfg.dtype == q.NF4_BF16 and cfg.dequant_repeats > 0 and all(
            r % 128 == 0 and c % 128 == 0 for _, r, c in cfg.per_block):
        out["matmul"] = matmul_block(q, torch, ls, f, cfg, stream, deq_ms / max(1, n_deq), set(keep))
    if args.protocol > 0:
        sub = ls.subset(keep)
        out["protocol"] = {
            "seconds_per_arm": args.protocol,
            "nf4_layer_error": protocol_arms(lambda: q.nf4_layer_error(ls, f, err, ws),
                                             args.protocol, torch, stream),
            "nf4_dequantize": protocol_arms(lambda: q.nf4_dequantize(sub, f, ws),
                                            args.protocol, torch, stream),
        }
        for k in ("nf4_layer_error", "nf4_dequantize"):
            pb = fused_bytes if k == "nf4_layer_error" else deq_bytes
            pm = 0.5 * (out["protocol"][k]["ms_A"] + out["protocol"][k]["ms_A2"])
            out["protocol"][k]["GBps"] = round(pb / (pm * 1e-3) / 1e9, 1)
    if not args.no_variants:   # last: it overwrites the stack's codes and outputs
        log("timing the codec variants")
        out["codec_variants"] = codec_variants(q, torch, ls, cfg, stream)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds, n_deq, n_total)
        log("timing the multi-threaded CPU pass")
        out["cpu_pass"] = cpu_pass(cfg, n_total)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
