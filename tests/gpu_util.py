"""Helpers for the GPU tests: move seeded inputs to the device, call the C ABI
through the binding, bring outputs back, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import quantized_lora_fine_nf4_amd as q

POISON = 0x5A


def layerset(ws_list, f, with_out=True, with_absmax=True) -> q.LayerSet:
    ls = q.LayerSet([int(w.size) for w in ws_list], f, with_out=with_out,
                    with_absmax=with_absmax)
    for i, w in enumerate(ws_list):
        ls.w_of(i).copy_(torch.from_numpy(np.ascontiguousarray(w, np.uint16).view(np.int16)))
    poison(ls)
    return ls


def poison(ls: q.LayerSet):
    """Fill every output buffer with a pattern, so unwritten bytes show."""
    for t in (ls.codes, ls.absmax, ls.qabsmax, ls.scale2, ls.out):
        if t is not None:
            t.view(torch.uint8).fill_(POISON)


def workspace(ns, f) -> torch.Tensor:
    return torch.empty(q.nf4_workspace_bytes(ns, f), dtype=torch.uint8, device="cuda")


def layer_error(ls, f, ws=None) -> torch.Tensor:
    ws = workspace(ls.ns, f) if ws is None else ws
    err = torch.full((len(ls),), float("nan"), dtype=torch.float64, device="cuda")
    q.nf4_layer_error(ls, f, err, ws)
    return err


def np_of(t: torch.Tensor, dtype) -> np.ndarray:
    return t.cpu().numpy().view(dtype)


def compare_layer(ls, i, w, dtype, dq, ref=None, check_absmax=True, check_out=False):
    """Bit-exact comparison of one layer's outputs with the oracle."""
    if ref is None:
        ref = oracle.layer_error(w, dtype, dq)
    codes = np_of(ls.codes_of(i), np.uint8)
    assert np.array_equal(codes, ref["codes"]), f"codes differ at {np.nonzero(codes != ref['codes'])[0][:10]}"
    if check_absmax and ls.absmax is not None:
        am = np_of(ls.absmax_of(i), np.uint32)
        assert np.array_equal(am, ref["absmax"].view(np.uint32)), "absmax differs"
    if dq:
        qa = np_of(ls.qabsmax_of(i), np.int8)
        assert np.array_equal(qa, ref["qabsmax"]), "qabsmax differs"
        s2 = np_of(ls.scale2_of(i), np.uint32)
        assert np.array_equal(s2, ref["scale2"].view(np.uint32)), "scale2 differs"
    if check_out:
        y = np_of(ls.out_of(i), np.uint16)
        bad = np.nonzero(y != ref["y"])[0]
        assert bad.size == 0, f"dequant differs at {bad[:10]}: {y[bad[:4]]} vs {ref['y'][bad[:4]]}"
    return ref


def rel_err(a: float, b: float) -> float:
    if a == b:
        return 0.0
    return abs(a - b) / max(abs(b), 1e-300)
