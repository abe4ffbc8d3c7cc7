"""Pins for the oracle's fused-consumer matmul (CPU only).

The matmul is numpy's fp64 product of exact values, so what needs pinning is
the wiring: orientation (x W^T forward, x W backward), the weight being the
codec's dequantised values, and row-major shapes.  Pins: a selector x picks
single rows / columns of W exactly; forward and backward agree through the
transpose identity x W^T = (W x^T)^T; the product equals an explicit triple
loop over exact Fractions on a tiny case.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

BF16 = oracle.BF16


def _weight(rows, cols, seed, dq):
    rng = np.random.default_rng(seed)
    w = oracle.to16_rne(rng.standard_normal(rows * cols).astype(np.float32) * 0.02, BF16)
    codes, absmax = oracle.quantize(w, BF16)
    if dq:
        q, s2 = oracle.double_quant(absmax)
        return codes, dict(qabsmax=q, scale2=s2)
    return codes, dict(absmax=absmax)


def _dequant(codes, rows, cols, consts):
    return oracle.from16(oracle.dequantize(codes, rows * cols, BF16, **consts),
                         BF16).astype(np.float64).reshape(rows, cols)


def _bits(a):
    return oracle.to16_rne(np.asarray(a, np.float32), BF16)


@pytest.mark.parametrize("dq", [False, True])
def test_selectors_pick_rows_and_columns(dq):
    rows, cols = 128, 192
    codes, consts = _weight(rows, cols, 1, dq)
    W = _dequant(codes, rows, cols, consts)
    # forward: x = e_j (over cols) gives column j of W for every output row n
    j = np.array([0, 5, 191])
    x = np.zeros((3, cols), np.float32)
    x[np.arange(3), j] = 1.0
    out = oracle.matmul(_bits(x), rows, cols, codes, BF16, backward=False, **consts)
    assert out.shape == (3, rows)
    assert np.array_equal(out, W[:, j].T)
    # backward: x = e_i (over rows) gives row i of W
    i = np.array([0, 77, 127])
    x = np.zeros((3, rows), np.float32)
    x[np.arange(3), i] = 1.0
    out = oracle.matmul(_bits(x), rows, cols, codes, BF16, backward=True, **consts)
    assert out.shape == (3, cols)
    assert np.array_equal(out, W[i, :])


def test_forward_backward_transpose_identity():
    """(x W^T)[a, n] = sum_k x[a, k] W[n, k]; with x = W itself (as bf16) the
    forward product is W W^T, symmetric, and its rows equal the backward
    product of W's rows with W^T's columns -- checked through both calls."""
    rows, cols = 128, 128
    codes, consts = _weight(rows, cols, 2, True)
    W = _dequant(codes, rows, cols, consts)
    wbits = _bits(W.astype(np.float32))
    fwd = oracle.matmul(wbits, rows, cols, codes, BF16, backward=False, **consts)
    assert np.allclose(fwd, fwd.T, rtol=0, atol=1e-15)
    bwd = oracle.matmul(wbits, rows, cols, codes, BF16, backward=True, **consts)   # W W (square)
    assert np.allclose(bwd, W @ W, rtol=0, atol=1e-15)


def test_tiny_case_equals_exact_triple_loop():
    rows, cols, m = 128, 128, 2
    codes, consts = _weight(rows, cols, 3, False)
    W = _dequant(codes, rows, cols, consts)
    rng = np.random.default_rng(4)
    xb = _bits(rng.standard_normal((m, cols)).astype(np.float32))
    x = oracle.from16(xb, BF16).reshape(m, cols)
    out = oracle.matmul(xb, rows, cols, codes, BF16, backward=False, **consts)
    for a in range(m):
        for n in (0, 63, 127):
            exact = sum(Fraction(float(x[a, k])) * Fraction(float(W[n, k])) for k in range(cols))
            assert abs(Fraction(float(out[a, n])) - exact) <= abs(exact) * Fraction(1, 1 << 50) + Fraction(1, 1 << 80)
