"""Binding of the host-CPU scoring pass (libnf4cpu.so, include/nf4_cpu.h).

The pass AQLoRA runs on the CPU ("AQLoRA" arXiv listing, English abstract),
on the host cores with OpenMP: same codes and constants as the GPU pass, bit
for bit, and the per-matrix reconstruction error.  A separate entry point for
comparison, never a fallback of the GPU calls.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .. import build as _build
from .. import nf4_format, nf4_layer, NF4Error, NF4_OK, BLOCK, DQ_GROUP

LIB_PATH = _build.CPU_LIB_PATH
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python quantized_lora_fine_nf4_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        L.nf4_cpu_layer_error.restype = ctypes.c_int
        L.nf4_cpu_layer_error.argtypes = [ctypes.c_void_p, ctypes.c_int32, nf4_format,
                                          ctypes.c_void_p, ctypes.c_int32]
        L.nf4_cpu_max_threads.restype = ctypes.c_int32
        L.nf4_cpu_max_threads.argtypes = []
        _lib = L
    return _lib


def max_threads() -> int:
    return int(lib().nf4_cpu_max_threads())


def layer_error(ws, f: nf4_format, threads: int = 0, with_absmax: bool = True) -> dict:
    """ws: list of uint16 arrays (16-bit patterns, one per matrix).
    -> dict(err, codes, absmax, qabsmax, scale2) of per-matrix lists."""
    dq = f.dq_group != 0
    ws = [np.ascontiguousarray(w, np.uint16).ravel() for w in ws]
    out = {"codes": [], "absmax": [], "qabsmax": [], "scale2": []}
    layers = []
    for w in ws:
        n = w.size
        nb = (n + BLOCK - 1) // BLOCK
        ng = (nb + DQ_GROUP - 1) // DQ_GROUP
        c = np.empty((n + 1) // 2, np.uint8)
        a = np.empty(nb, np.float32) if (with_absmax or not dq) else None
        qa = np.empty(nb, np.int8) if dq else None
        s2 = np.empty(ng, np.float32) if dq else None
        for k, v in (("codes", c), ("absmax", a), ("qabsmax", qa), ("scale2", s2)):
            out[k].append(v)
        p = lambda x: None if x is None else x.ctypes.data
        layers.append(nf4_layer(n, p(w), p(c), p(a), p(qa), p(s2), None))
    arr = (nf4_layer * len(layers))(*layers)
    err = np.empty(len(ws), np.float64)
    st = lib().nf4_cpu_layer_error(arr, len(ws), f, err.ctypes.data, int(threads))
    if st != NF4_OK:
        raise NF4Error(st, "nf4_cpu_layer_error")
    out["err"] = err
    out["_keep"] = ws
    return out
