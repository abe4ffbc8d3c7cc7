"""Seeded synthetic weight stacks (input generation only; no codec arithmetic).

ctypes wrapper over ``libsynth.so`` (``synth.c``).  Every layer is
reproducible from (config id, layer index); any 4096-aligned slice of a layer
can be regenerated alone, which lets full-size tests check sampled tiles.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .configs import CONFIGS, BY_NAME, StackConfig, GIB, BF16, FP16, NORMAL, STUDENT_T4  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
CHUNK = 4096


def build() -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", LIB_PATH + ".tmp", os.path.join(_HERE, "synth.c"), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        u64, i64, f64, i32, P = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_double,
                                 ctypes.c_int, ctypes.c_void_p)
        L.synth_layer_seed.restype = u64
        L.synth_layer_seed.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
        L.synth_layer_sigma.restype = f64
        L.synth_layer_sigma.argtypes = [u64, f64, f64]
        L.synth_outlier_positions.restype = i64
        L.synth_outlier_positions.argtypes = [u64, i64, f64, f64, f64, P]
        L.synth_generate.restype = i32
        L.synth_generate.argtypes = [u64, i64, i32, f64, f64, f64, f64, i32, i64, i64, P, i32]
        _lib = L
    return _lib


def default_threads() -> int:
    # at most 16 threads: a GPU host may give a process 16 CPUs whatever os.cpu_count() reports
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def layer_seed(cfg: StackConfig, i: int) -> int:
    return lib().synth_layer_seed(cfg.cid, i)


def layer_sigma(cfg: StackConfig, i: int) -> float:
    return lib().synth_layer_sigma(layer_seed(cfg, i), cfg.sigma_lo, cfg.sigma_hi)


def outlier_positions(cfg: StackConfig, i: int) -> np.ndarray:
    n = cfg.n(i)
    m = int(round(cfg.outlier_frac * n))
    out = np.empty(max(m, 1), np.int64)
    k = lib().synth_outlier_positions(layer_seed(cfg, i), n, cfg.outlier_frac,
                                      cfg.sigma_lo, cfg.sigma_hi, out.ctypes.data)
    return out[:k]


def generate_into(cfg: StackConfig, i: int, out_ptr: int, first: int = 0,
                  count: int | None = None, threads: int | None = None) -> None:
    """Write elements [first, first+count) of layer i (uint16 bits) to out_ptr."""
    n = cfg.n(i)
    if count is None:
        count = n - first
    rc = lib().synth_generate(layer_seed(cfg, i), n, cfg.dist, cfg.sigma_lo, cfg.sigma_hi,
                              cfg.outlier_frac, cfg.outlier_scale, cfg.dtype,
                              first, count, out_ptr, threads or default_threads())
    if rc != 0:
        raise ValueError(f"bad slice [{first}, {first}+{count}) of a {n}-element layer")


def generate(cfg: StackConfig, i: int, first: int = 0, count: int | None = None,
             threads: int | None = None) -> np.ndarray:
    n = cfg.n(i)
    if count is None:
        count = n - first
    out = np.empty(count, np.uint16)
    generate_into(cfg, i, out.ctypes.data, first, count, threads)
    return out


def generate_raw(seed: int, n: int, dtype: int = BF16, dist: int = NORMAL,
                 sigma: float = 0.02, outlier_frac: float = 0.0,
                 outlier_scale: float = 10.0, threads: int = 1) -> np.ndarray:
    """A free-standing seeded matrix (for tests of arbitrary n)."""
    out = np.empty(n, np.uint16)
    rc = lib().synth_generate(seed, n, dist, sigma, 0.0, outlier_frac, outlier_scale,
                              dtype, 0, n, out.ctypes.data, threads)
    assert rc == 0
    return out


def fill_device(cfg: StackConfig, views, threads: int | None = None,
                staging_elems: int = 1 << 26, progress=None) -> None:
    """Generate every layer of ``cfg`` on the host and copy it into the
    matching device tensor of ``views`` (int16 bit patterns, one per layer),
    through two pinned staging buffers so generation overlaps the copies."""
    import torch
    bufs = [torch.empty(staging_elems, dtype=torch.int16, pin_memory=True) for _ in range(2)]
    events = [None, None]
    stream = torch.cuda.current_stream()
    k = 0
    for i in range(cfg.n_layers):
        n = cfg.n(i)
        assert views[i].numel() == n and views[i].dtype == torch.int16
        for first in range(0, n, staging_elems):
            cnt = min(staging_elems, n - first)
            b = k % 2
            if events[b] is not None:
                events[b].synchronize()
            generate_into(cfg, i, bufs[b].data_ptr(), first, cnt, threads)
            views[i][first:first + cnt].copy_(bufs[b][:cnt], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(stream)
            events[b] = ev
            k += 1
        if progress is not None:
            progress(i)
    torch.cuda.synchronize()
