"""MI355X-native NF4 weight codec and AQLoRA layer selector.

Thin Python binding over ``libnf4.so`` (C ABI: ``include/nf4.h``).  The
functions carry the C names and only marshal arguments: every step of the
codec and of the ranking runs in the HIP kernels.  PyTorch provides device
memory and the current stream; nothing here computes on the CPU, and a
missing library raises instead of falling back.

    nf4_quantize, nf4_double_quant, nf4_dequantize, nf4_dequantize_masked,
    nf4_layer_error, aqlora_select_topk     -- enqueue on the current stream
    nf4_workspace_bytes, aqlora_workspace_bytes, nf4_storage_bytes,
    aqlora_promote_cost, nf4_levels, nf4_thresholds, nf4_abi_version
                                            -- host-only helpers

``LayerSet`` allocates the per-layer device buffers of a stack of matrices
(one tensor per buffer kind, per-layer slices aligned as the ABI requires)
and keeps the matching ``nf4_layer`` array.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnf4.so")

NF4_OK, NF4_E_ARG, NF4_E_ALIGN, NF4_E_UNSUPPORTED, NF4_E_WORKSPACE, NF4_E_HIP = range(6)
NF4_BF16, NF4_FP16 = 0, 1
AQLORA_PREFIX, AQLORA_FILL = 0, 1
BLOCK, DQ_GROUP = 64, 256


class NF4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib_or_none().nf4_status_str(status).decode() if _lib_or_none() else str(status)
        extra = ""
        if status == NF4_E_HIP and _lib_or_none():
            extra = f" (hipError {_lib_or_none().nf4_last_hip_error()})"
        super().__init__(f"{where}: {msg}{extra}")


class nf4_format(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("blocksize", ctypes.c_int32),
                ("dq_group", ctypes.c_int32)]


class nf4_variant(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("blocksize", ctypes.c_int32),
                ("dq_kind", ctypes.c_int32)]


NF4_DQ_NONE, NF4_DQ_INT8, NF4_DQ_INT8_MEAN, NF4_DQ_E4M3_MEAN = range(4)


class nf4_layer(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("w", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("absmax", ctypes.c_void_p), ("qabsmax", ctypes.c_void_p),
                ("scale2", ctypes.c_void_p), ("out", ctypes.c_void_p)]


EXPORTS = {
    # name: (restype, argtypes)
    "nf4_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, nf4_format, ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]),
    "nf4_double_quant": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, nf4_format,
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "nf4_dequantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, nf4_format,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "nf4_dequantize_masked": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, nf4_format,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                             ctypes.c_void_p]),
    "nf4_layer_error": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, nf4_format,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]),
    "nf4_layer_error_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, nf4_format,
                                               ctypes.c_void_p, ctypes.c_void_p]),
    "nf4_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "nf4_layer_error_norm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, nf4_format,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_size_t, ctypes.c_void_p]),
    "aqlora_select_topk": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_void_p]),
    "aqlora_select": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                     ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]),
    "nf4_matmul": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, nf4_format,
                                  ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    "nf4_matmul_ws": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, nf4_format,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]),
    "nf4_matmul_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                                     ctypes.c_int64]),
    "nf4_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_void_p, nf4_format]),
    "nf4_layer_error_variant": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, nf4_variant,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_size_t, ctypes.c_void_p]),
    "nf4_dequantize_variant": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, nf4_variant,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                              ctypes.c_void_p]),
    "nf4_workspace_bytes_variant": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_void_p,
                                                      nf4_variant]),
    "nf4_storage_bytes_variant": (ctypes.c_int64, [ctypes.c_int64, nf4_variant]),
    "aqlora_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32]),
    "nf4_storage_bytes": (ctypes.c_int64, [ctypes.c_int64, nf4_format]),
    "aqlora_promote_cost": (ctypes.c_int64, [ctypes.c_int64, nf4_format]),
    "nf4_levels": (None, [ctypes.c_void_p]),
    "nf4_thresholds": (None, [ctypes.c_void_p]),
    "nf4_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "nf4_abi_version": (ctypes.c_int32, []),
    "nf4_last_hip_error": (ctypes.c_int32, []),
}

_lib = None


def _lib_or_none():
    return _lib


def lib() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python quantized_lora_fine_nf4_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def fmt(dtype: int = NF4_BF16, dq: bool = True) -> nf4_format:
    return nf4_format(int(dtype), BLOCK, DQ_GROUP if dq else 0)


def _ptr(t) -> int | None:
    if t is None:
        return None
    return int(t.data_ptr())


def _stream(stream) -> int | None:
    if stream is not None:
        return int(stream) if isinstance(stream, int) else int(stream.cuda_stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _check(status: int, where: str):
    if status != NF4_OK:
        raise NF4Error(status, where)


def _layers_arg(layers):
    """A LayerSet / LayerSubset, or a sequence of nf4_layer structs."""
    if isinstance(layers, (LayerSet, LayerSubset)):
        return ctypes.byref(layers.c_layers), len(layers)
    arr = (nf4_layer * len(layers))(*layers)
    return arr, len(layers)


# ---- the five calls -------------------------------------------------------

def nf4_quantize(layers, f: nf4_format, ws, stream=None) -> None:
    arr, nl = _layers_arg(layers)
    _check(lib().nf4_quantize(arr, nl, f, _ptr(ws), ws.numel() * ws.element_size(),
                              _stream(stream)), "nf4_quantize")


def nf4_double_quant(layers, f: nf4_format, ws, stream=None) -> None:
    arr, nl = _layers_arg(layers)
    _check(lib().nf4_double_quant(arr, nl, f, _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "nf4_double_quant")


def nf4_dequantize(layers, f: nf4_format, ws, stream=None) -> None:
    arr, nl = _layers_arg(layers)
    _check(lib().nf4_dequantize(arr, nl, f, _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)), "nf4_dequantize")


def nf4_dequantize_masked(layers, f: nf4_format, skip, ws, stream=None) -> None:
    """nf4_dequantize of the layers whose byte in skip (device uint8[nl], e.g.
    aqlora_select_topk's selected) is 0; the others' outputs are untouched."""
    arr, nl = _layers_arg(layers)
    _check(lib().nf4_dequantize_masked(arr, nl, f, _ptr(skip), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream)), "nf4_dequantize_masked")


def nf4_layer_error(layers, f: nf4_format, err, ws, stream=None) -> None:
    arr, nl = _layers_arg(layers)
    _check(lib().nf4_layer_error(arr, nl, f, _ptr(err), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)),
           "nf4_layer_error")


def nf4_layer_error_noalloc(layers, f: nf4_format, err, stream=None) -> None:
    """nf4_layer_error with the library's fixed per-device scratch instead of
    a workspace (for callers that cannot allocate)."""
    arr, nl = _layers_arg(layers)
    _check(lib().nf4_layer_error_noalloc(arr, nl, f, _ptr(err), _stream(stream)),
           "nf4_layer_error_noalloc")


def nf4_noalloc_scratch_bytes() -> int:
    return int(lib().nf4_noalloc_scratch_bytes())


def aqlora_select_topk(err, cost, budget_bytes: int, k_cap: int, selected, k_out, ws,
                       stream=None) -> None:
    nl = int(err.numel())
    _check(lib().aqlora_select_topk(_ptr(err), _ptr(cost), nl, int(budget_bytes), int(k_cap),
                                    _ptr(selected), _ptr(k_out), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)),
           "aqlora_select_topk")


def nf4_layer_error_norm(layers, f: nf4_format, err, sumsq, ws, stream=None) -> None:
    arr, nl = _layers_arg(layers)
    _check(lib().nf4_layer_error_norm(arr, nl, f, _ptr(err), _ptr(sumsq), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)),
           "nf4_layer_error_norm")


def aqlora_select(err, cost, budget_bytes: int, k_cap: int, selected, k_out, ws, denom=None,
                  group_end=None, rule: int = AQLORA_PREFIX, stream=None) -> None:
    """group_end: host sequence of group ends (copied before return), or None."""
    nl = int(err.numel())
    ge = None if group_end is None else np.ascontiguousarray(group_end, np.int32)
    _check(lib().aqlora_select(_ptr(err), _ptr(denom), _ptr(cost), nl,
                               None if ge is None else ge.ctypes.data,
                               0 if ge is None else int(ge.size), int(budget_bytes), int(k_cap),
                               int(rule), _ptr(selected), _ptr(k_out), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)),
           "aqlora_select")


def nf4_matmul(layer, rows: int, cols: int, f: nf4_format, x, out, backward: bool = False,
               stream=None) -> None:
    """out = x @ W^T (forward) or x @ W (backward) with W in NF4 form.
    layer: an nf4_layer struct (e.g. ls.c_layers[i]); x, out: device tensors
    (x in the 16-bit type f.dtype names; out float32 or that 16-bit type)."""
    import torch
    m = int(x.shape[0]) if x.dim() > 1 else 1
    out_fp32 = 1 if out.dtype == torch.float32 else 0
    _check(lib().nf4_matmul(ctypes.byref(layer), int(rows), int(cols), f, int(bool(backward)),
                            _ptr(x), m, _ptr(out), out_fp32, _stream(stream)), "nf4_matmul")


def nf4_matmul_workspace_bytes(rows: int, cols: int, backward: bool, m: int) -> int:
    return int(lib().nf4_matmul_workspace_bytes(int(rows), int(cols), int(bool(backward)), int(m)))


def nf4_matmul_ws(layer, rows: int, cols: int, f: nf4_format, x, out, ws, backward: bool = False,
                  stream=None) -> None:
    """nf4_matmul with a workspace (ws: device uint8 tensor of at least
    nf4_matmul_workspace_bytes(...) bytes, or None when that is 0): the
    few-token forward kernel at m <= 32, the split reduction when the output
    tiles alone do not fill the GPU, and the split of the tiles left over
    after whole rounds of large tiles."""
    import torch
    m = int(x.shape[0]) if x.dim() > 1 else 1
    out_fp32 = 1 if out.dtype == torch.float32 else 0
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().nf4_matmul_ws(ctypes.byref(layer), int(rows), int(cols), f, int(bool(backward)),
                               _ptr(x), m, _ptr(out), out_fp32, _ptr(ws), nbytes, _stream(stream)),
           "nf4_matmul_ws")


def variant(dtype: int = NF4_BF16, block: int = BLOCK, kind: int = NF4_DQ_INT8) -> nf4_variant:
    return nf4_variant(int(dtype), int(block), int(kind))


def nf4_layer_error_variant(layers, v: nf4_variant, err, ws, mean=None, stream=None) -> None:
    arr, nl = _layers_arg(layers)
    _check(lib().nf4_layer_error_variant(arr, nl, v, _ptr(mean), _ptr(err), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)),
           "nf4_layer_error_variant")


def nf4_dequantize_variant(layers, v: nf4_variant, ws, mean=None, stream=None) -> None:
    arr, nl = _layers_arg(layers)
    _check(lib().nf4_dequantize_variant(arr, nl, v, _ptr(mean), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)),
           "nf4_dequantize_variant")


def nf4_workspace_bytes_variant(ns, v: nf4_variant) -> int:
    a = np.ascontiguousarray(ns, np.int64)
    return int(lib().nf4_workspace_bytes_variant(a.size, a.ctypes.data if a.size else None, v))


def nf4_storage_bytes_variant(n: int, v: nf4_variant) -> int:
    return int(lib().nf4_storage_bytes_variant(int(n), v))


# ---- host helpers ---------------------------------------------------------

def nf4_workspace_bytes(ns, f: nf4_format) -> int:
    a = np.ascontiguousarray(ns, np.int64)
    return int(lib().nf4_workspace_bytes(a.size, a.ctypes.data, f))


def aqlora_workspace_bytes(nl: int) -> int:
    return int(lib().aqlora_workspace_bytes(nl))


def nf4_storage_bytes(n: int, f: nf4_format) -> int:
    return int(lib().nf4_storage_bytes(n, f))


def aqlora_promote_cost(n: int, f: nf4_format) -> int:
    return int(lib().aqlora_promote_cost(n, f))


def nf4_levels() -> np.ndarray:
    out = np.zeros(16, np.float32)
    lib().nf4_levels(out.ctypes.data)
    return out


def nf4_thresholds() -> np.ndarray:
    out = np.zeros(15, np.float32)
    lib().nf4_thresholds(out.ctypes.data)
    return out


def nf4_abi_version() -> int:
    return int(lib().nf4_abi_version())


# ---- device buffers for a stack of matrices -------------------------------

def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


class LayerSet:
    """Device buffers for ``len(ns)`` matrices of ``ns[i]`` elements.

    Each buffer kind is one tensor; layer i's slice starts at an offset that
    keeps the ABI's alignment (weights, codes and outputs 16 B).
    Attributes: ``w`` (int16 bits), ``codes`` (uint8), ``absmax`` (float32),
    ``qabsmax`` (int8), ``scale2`` (float32), ``out`` (int16 bits), the offset
    lists ``*_off``, and ``c_layers`` (the nf4_layer array).  ``w``, ``codes``
    and ``out`` may be given (e.g. another LayerSet's, whose offsets do not
    depend on the block size) instead of allocated.
    """

    def __init__(self, ns, f: nf4_format, device="cuda", with_out: bool = True,
                 with_absmax: bool = True, w=None, block: int = BLOCK, codes=None, out=None):
        import torch
        self.ns = [int(n) for n in ns]
        self.fmt = f
        dq = f.dq_group != 0
        self.block = int(block)
        nb = [(n + self.block - 1) // self.block for n in self.ns]
        ng = [(b + DQ_GROUP - 1) // DQ_GROUP for b in nb]

        def offsets(sizes, align):
            offs, run = [], 0
            for s in sizes:
                offs.append(run)
                run += _round_up(max(s, 1), align)
            return offs, run

        self.w_off, wtot = offsets(self.ns, 64)
        self.c_off, ctot = offsets([(n + 1) // 2 for n in self.ns], 64)
        self.a_off, atot = offsets(nb, 64)
        self.s_off, stot = offsets(ng, 64)
        if w is None:
            self.w = torch.empty(wtot, dtype=torch.int16, device=device)
        else:
            assert w.dtype == torch.int16 and w.numel() >= wtot
            self.w = w
        if codes is None:
            self.codes = torch.empty(ctot, dtype=torch.uint8, device=device)
        else:
            assert codes.dtype == torch.uint8 and codes.numel() >= ctot
            self.codes = codes
        self.absmax = torch.empty(atot, dtype=torch.float32, device=device) if (with_absmax or not dq) else None
        self.qabsmax = torch.empty(atot, dtype=torch.int8, device=device) if dq else None
        self.scale2 = torch.empty(stot, dtype=torch.float32, device=device) if dq else None
        if out is not None:
            assert out.dtype == torch.int16 and out.numel() >= wtot
            self.out = out
        else:
            self.out = torch.empty(wtot, dtype=torch.int16, device=device) if with_out else None
        self._build()

    def _build(self):
        L = []
        for i, n in enumerate(self.ns):
            def at(t, off, esz):
                return None if t is None else int(t.data_ptr()) + off * esz
            L.append(nf4_layer(n, at(self.w, self.w_off[i], 2), at(self.codes, self.c_off[i], 1),
                               at(self.absmax, self.a_off[i], 4), at(self.qabsmax, self.a_off[i], 1),
                               at(self.scale2, self.s_off[i], 4), at(self.out, self.w_off[i], 2)))
        self.c_layers = (nf4_layer * len(L))(*L)

    def subset(self, idx) -> "LayerSubset":
        return LayerSubset(self, list(idx))

    def __len__(self):
        return len(self.ns)

    # per-layer views
    def w_of(self, i):
        return self.w[self.w_off[i]: self.w_off[i] + self.ns[i]]

    def out_of(self, i):
        return self.out[self.w_off[i]: self.w_off[i] + self.ns[i]]

    def codes_of(self, i):
        return self.codes[self.c_off[i]: self.c_off[i] + (self.ns[i] + 1) // 2]

    def absmax_of(self, i):
        nb = (self.ns[i] + self.block - 1) // self.block
        return self.absmax[self.a_off[i]: self.a_off[i] + nb]

    def qabsmax_of(self, i):
        nb = (self.ns[i] + self.block - 1) // self.block
        return self.qabsmax[self.a_off[i]: self.a_off[i] + nb]

    def scale2_of(self, i):
        ng = ((self.ns[i] + self.block - 1) // self.block + DQ_GROUP - 1) // DQ_GROUP
        return self.scale2[self.s_off[i]: self.s_off[i] + ng]


class LayerSubset:
    """Some layers of a LayerSet, e.g. the ones left in NF4 after promotion."""

    def __init__(self, parent: LayerSet, idx):
        self.parent = parent
        self.idx = idx
        self.c_layers = (nf4_layer * len(idx))(*[parent.c_layers[i] for i in idx])

    def __len__(self):
        return len(self.idx)

