"""CPU oracle for the NF4 codec and the AQLoRA ranking -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
``quantized_lora_fine_nf4_amd``) never imports it and shares no code with it.

Thin ctypes wrapper over ``liboracle_nf4.so`` (plain single-threaded C, see
``nf4_oracle.c`` for every step and the passage of the pages it follows).
Arrays are numpy; 16-bit weights travel as ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle_nf4.so")
SOURCES = [os.path.join(_HERE, "nf4_oracle.c")]

BF16, FP16 = 0, 1
BLOCK, DQ_GROUP = 64, 256


BUILD_FLAGS = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math"]


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = [*BUILD_FLAGS, "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp",
           *SOURCES, "-lm"]
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
        P = ctypes.c_void_p
        i64, i32, f32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
        sigs = {
            "nf4o_levels": (i32, [P]),
            "nf4o_thresholds": (None, [P]),
            "nf4o_from16": (f32, [ctypes.c_uint16, i32]),
            "nf4o_to16_rne": (ctypes.c_uint16, [f32, i32]),
            "nf4o_to16_rne_array": (None, [P, i64, i32, P]),
            "nf4o_encode": (i32, [f32]),
            "nf4o_encode_array": (None, [P, i64, P]),
            "nf4o_quantize": (None, [P, i64, i32, P, P]),
            "nf4o_double_quant": (None, [P, i64, P, P]),
            "nf4o_dequantize": (None, [P, i64, i32, P, P, P, P]),
            "nf4o_sse": (f64, [P, P, i64, i32]),
            "nf4o_layer_error": (f64, [P, i64, i32, i32, P, P, P, P, P]),
            "nf4o_storage_bytes": (i64, [i64, i32]),
            "nf4o_promote_cost": (i64, [i64, i32]),
            "nf4o_select_topk": (i32, [P, P, i32, i64, i32, P]),
            "nf4o_sumsq": (ctypes.c_double, [P, i64, i32]),
            "nf4o_e4m3_decode": (ctypes.c_float, [ctypes.c_uint8]),
            "nf4o_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
            "nf4o_storage_bytes_ex": (i64, [i64, i32, i32]),
            "nf4o_layer_error_ex": (ctypes.c_double, [P, i64, i32, i32, i32, P, P, P, P, P, P]),
            "nf4o_select": (i32, [P, P, P, i32, P, i32, i64, i32, i32, P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def nblocks(n: int) -> int:
    return (n + BLOCK - 1) // BLOCK


def ngroups(n: int) -> int:
    return (nblocks(n) + DQ_GROUP - 1) // DQ_GROUP


def levels() -> np.ndarray:
    out = np.zeros(16, np.float32)
    lib().nf4o_levels(_p(out))
    return out


def thresholds() -> np.ndarray:
    out = np.zeros(15, np.float32)
    lib().nf4o_thresholds(_p(out))
    return out


def from16(h: np.ndarray, dtype: int) -> np.ndarray:
    """16-bit bit patterns -> float32 values (exact)."""
    h = np.ascontiguousarray(h, np.uint16)
    if dtype == BF16:
        return (h.astype(np.uint32) << 16).view(np.float32)
    return h.view(np.float16).astype(np.float32)


def to16_rne(f: np.ndarray, dtype: int) -> np.ndarray:
    f = np.ascontiguousarray(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().nf4o_to16_rne_array(_p(f), f.size, dtype, _p(out))
    return out


def encode(s: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(s, np.float32)
    out = np.empty(s.shape, np.uint8)
    lib().nf4o_encode_array(_p(s), s.size, _p(out))
    return out


def quantize(w: np.ndarray, dtype: int):
    """-> (codes[ceil(n/2)] u8, absmax[nb] f32)."""
    w = np.ascontiguousarray(w, np.uint16).ravel()
    n = w.size
    codes = np.empty((n + 1) // 2, np.uint8)
    absmax = np.empty(nblocks(n), np.float32)
    lib().nf4o_quantize(_p(w), n, dtype, _p(codes), _p(absmax))
    return codes, absmax


def double_quant(absmax: np.ndarray):
    """-> (qabsmax[nb] i8, scale2[ceil(nb/256)] f32)."""
    absmax = np.ascontiguousarray(absmax, np.float32)
    nb = absmax.size
    q = np.empty(nb, np.int8)
    s2 = np.empty((nb + DQ_GROUP - 1) // DQ_GROUP, np.float32)
    lib().nf4o_double_quant(_p(absmax), nb, _p(q), _p(s2))
    return q, s2


def dequantize(codes, n: int, dtype: int, absmax=None, qabsmax=None, scale2=None):
    codes = np.ascontiguousarray(codes, np.uint8)
    out = np.empty(n, np.uint16)
    absmax = None if absmax is None else np.ascontiguousarray(absmax, np.float32)
    qabsmax = None if qabsmax is None else np.ascontiguousarray(qabsmax, np.int8)
    scale2 = None if scale2 is None else np.ascontiguousarray(scale2, np.float32)
    lib().nf4o_dequantize(_p(codes), n, dtype, _p(absmax), _p(qabsmax), _p(scale2), _p(out))
    return out


def sse(w: np.ndarray, y: np.ndarray, dtype: int) -> float:
    w = np.ascontiguousarray(w, np.uint16).ravel()
    y = np.ascontiguousarray(y, np.uint16).ravel()
    assert w.size == y.size
    return lib().nf4o_sse(_p(w), _p(y), w.size, dtype)


def layer_error(w: np.ndarray, dtype: int, dq: bool):
    """The whole scoring pass for one matrix.

    -> dict(err, codes, absmax, qabsmax, scale2, y)."""
    w = np.ascontiguousarray(w, np.uint16).ravel()
    n = w.size
    codes = np.empty((n + 1) // 2, np.uint8)
    absmax = np.empty(nblocks(n), np.float32)
    q = np.empty(nblocks(n), np.int8) if dq else None
    s2 = np.empty(ngroups(n), np.float32) if dq else None
    y = np.empty(n, np.uint16)
    err = lib().nf4o_layer_error(_p(w), n, dtype, int(dq), _p(codes), _p(absmax),
                                 _p(q), _p(s2), _p(y))
    return dict(err=err, codes=codes, absmax=absmax, qabsmax=q, scale2=s2, y=y)


def storage_bytes(n: int, dq: bool) -> int:
    return lib().nf4o_storage_bytes(n, int(dq))


def promote_cost(n: int, dq: bool) -> int:
    return lib().nf4o_promote_cost(n, int(dq))


def select_topk(err, cost, budget: int = -1, kcap: int = -1):
    """-> (selected[nl] u8, K)."""
    err = np.ascontiguousarray(err, np.float64)
    cost = np.ascontiguousarray(cost, np.int64)
    nl = err.size
    sel = np.zeros(nl, np.uint8)
    K = lib().nf4o_select_topk(_p(err), _p(cost), nl, int(budget), int(kcap), _p(sel))
    return sel, K


def sumsq(w: np.ndarray, dtype: int) -> float:
    """Sum of x^2 over a 16-bit matrix, fp64."""
    w = np.ascontiguousarray(w, np.uint16).ravel()
    return lib().nf4o_sumsq(_p(w), w.size, dtype)


PREFIX, FILL = 0, 1


def select(err, cost, budget: int = -1, kcap: int = -1, denom=None, group_end=None,
           rule: int = PREFIX):
    """General selection -> (selected[nl] u8, units taken)."""
    err = np.ascontiguousarray(err, np.float64)
    cost = np.ascontiguousarray(cost, np.int64)
    nl = err.size
    d = None if denom is None else np.ascontiguousarray(denom, np.float64)
    g = None if group_end is None else np.ascontiguousarray(group_end, np.int32)
    sel = np.zeros(nl, np.uint8)
    K = lib().nf4o_select(_p(err), _p(d), _p(cost), nl, _p(g), 0 if g is None else g.size,
                          int(budget), int(kcap), int(rule), _p(sel))
    return sel, K


def matmul(x_bits, rows: int, cols: int, codes, dtype: int = BF16, absmax=None, qabsmax=None,
           scale2=None, backward: bool = False) -> np.ndarray:
    """The matmul that consumes an NF4 weight, in fp64: W [rows x cols] is
    dequantised by the oracle (the 16-bit values nf4o_dequantize defines),
    then forward x[m x cols] @ W^T, backward x[m x rows] @ W.  x_bits: 16-bit
    patterns of x.  The product is numpy's fp64 matmul of the exact values."""
    w = from16(dequantize(codes, rows * cols, dtype, absmax, qabsmax, scale2), dtype)
    w = w.astype(np.float64).reshape(rows, cols)
    x = from16(np.ascontiguousarray(x_bits, np.uint16), dtype).astype(np.float64)
    x = x.reshape(-1, rows if backward else cols)
    return x @ w if backward else x @ w.T


KIND_NONE, KIND_INT8, KIND_INT8_MEAN, KIND_FP8_MEAN = 0, 1, 2, 3


def e4m3_decode(b: int) -> float:
    return float(lib().nf4o_e4m3_decode(int(b)))


def e4m3_encode(v: float) -> int:
    return int(lib().nf4o_e4m3_encode(float(v)))


def storage_bytes_ex(n: int, block: int, kind: int) -> int:
    return int(lib().nf4o_storage_bytes_ex(int(n), int(block), int(kind)))


def layer_error_ex(w: np.ndarray, dtype: int, block: int, kind: int) -> dict:
    """Variant codec pass for one matrix -> dict(err, codes, absmax, q, scale2, mean, y)."""
    w = np.ascontiguousarray(w, np.uint16).ravel()
    n = w.size
    nb = (n + block - 1) // block
    ng = (nb + DQ_GROUP - 1) // DQ_GROUP
    codes = np.empty((n + 1) // 2, np.uint8)
    absmax = np.empty(nb, np.float32)
    qv = np.zeros(nb, np.uint8)
    s2 = np.zeros(ng, np.float32)
    mean = np.zeros(1, np.float32)
    y = np.empty(n, np.uint16)
    err = lib().nf4o_layer_error_ex(_p(w), n, dtype, block, kind, _p(codes), _p(absmax), _p(qv),
                                    _p(s2), _p(mean), _p(y))
    return dict(err=err, codes=codes, absmax=absmax, q=qv, scale2=s2, mean=float(mean[0]), y=y)
