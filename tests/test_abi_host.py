"""C ABI contract on the host: symbols, helpers, argument errors (no GPU needed).

Every argument check runs before any HIP call, so the error paths are
exercised here with stand-in (never dereferenced) pointers.
"""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
import quantized_lora_fine_nf4_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 256-aligned stand-in address; no call below reaches the device


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "nf4.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("nf4_", "aqlora_"))))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 14, names
    L = ctypes.CDLL(q.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(q.EXPORTS), set(names) ^ set(q.EXPORTS)
    assert q.nf4_abi_version() == 5


def test_embedded_levels_and_thresholds_equal_the_oracles():
    assert np.array_equal(q.nf4_levels().view(np.uint32), oracle.levels().view(np.uint32))
    assert np.array_equal(q.nf4_thresholds().view(np.uint32), oracle.thresholds().view(np.uint32))


def test_storage_and_cost_helpers_match_oracle():
    rng = np.random.default_rng(0)
    ns = [1, 2, 63, 64, 65, 127, 16383, 16384, 16385, 64 * 257, 4096 * 4096, 70_778_880]
    ns += list(rng.integers(1, 10**9, 50))
    for n in ns:
        for dq in (False, True):
            f = q.fmt(q.NF4_BF16, dq)
            assert q.nf4_storage_bytes(int(n), f) == oracle.storage_bytes(int(n), dq)
            assert q.aqlora_promote_cost(int(n), f) == oracle.promote_cost(int(n), dq)
    assert q.nf4_storage_bytes(0, q.fmt()) == -1
    assert q.nf4_storage_bytes(10, q.nf4_format(0, 32, 0)) == -1


def test_workspace_sizes():
    f = q.fmt()
    ns = [16384 * 3 + 1, 100, 64]
    tiles = 4 + 1 + 1
    # layer table (64 B per matrix) + an 8-byte record per tile of 16384 weights +
    # 4 fp64 error partials and 4 fp64 sum-of-squares partials per tile
    assert q.nf4_workspace_bytes(ns, f) == (256 + ((tiles * 8 + 255) // 256) * 256
                                            + 2 * (((tiles * 4 * 8 + 255) // 256) * 256))
    assert q.nf4_workspace_bytes([], f) == 0
    assert q.nf4_workspace_bytes([0], f) == 0
    # rank, perm, staged group ends (int32), unit scores, unit costs (8 B), flags (1 B)
    assert q.aqlora_workspace_bytes(280) == 3 * 1280 + 2 * 2304 + 512
    assert q.aqlora_workspace_bytes(0) == 0
    assert q.aqlora_workspace_bytes(65537) == 0


def _L(n=128, w=FAKE, codes=FAKE, absmax=FAKE, qabsmax=FAKE, scale2=FAKE, out=FAKE):
    return q.nf4_layer(n, w, codes, absmax, qabsmax, scale2, out)


def _call(name, layers, f, ws=FAKE, ws_bytes=1 << 20, err=FAKE, skip=FAKE):
    L = q.lib()
    arr = (q.nf4_layer * max(1, len(layers)))(*layers)
    if name == "nf4_layer_error":
        return L.nf4_layer_error(arr, len(layers), f, err, ws, ws_bytes, None)
    if name == "nf4_dequantize_masked":
        return L.nf4_dequantize_masked(arr, len(layers), f, skip, ws, ws_bytes, None)
    return getattr(L, name)(arr, len(layers), f, ws, ws_bytes, None)


CODEC = ["nf4_quantize", "nf4_double_quant", "nf4_dequantize", "nf4_dequantize_masked", "nf4_layer_error"]


@pytest.mark.parametrize("name", CODEC)
def test_unsupported_formats(name):
    for f in (q.nf4_format(0, 32, 256), q.nf4_format(0, 64, 128), q.nf4_format(2, 64, 0)):
        assert _call(name, [_L()], f) == q.NF4_E_UNSUPPORTED
    if name == "nf4_double_quant":
        assert _call(name, [_L()], q.fmt(dq=False)) == q.NF4_E_UNSUPPORTED


@pytest.mark.parametrize("name", CODEC)
def test_bad_layers(name):
    f = q.fmt()
    assert _call(name, [], f) == q.NF4_E_ARG
    assert _call(name, [_L(n=0)], f) == q.NF4_E_ARG
    assert _call(name, [_L(n=-5)], f) == q.NF4_E_ARG
    assert _call(name, [_L(n=1 << 40)], f) == q.NF4_E_ARG
    assert _call(name, [_L(), _L(n=0)], f) == q.NF4_E_ARG
    need = {"nf4_quantize": ["w", "codes", "absmax", "qabsmax", "scale2"],
            "nf4_double_quant": ["absmax", "qabsmax", "scale2"],
            "nf4_dequantize": ["codes", "qabsmax", "scale2", "out"],
            "nf4_dequantize_masked": ["codes", "qabsmax", "scale2", "out"],
            "nf4_layer_error": ["w", "codes", "qabsmax", "scale2"]}[name]
    for field in need:
        assert _call(name, [_L(**{field: None})], f) == q.NF4_E_ARG, field
    if name == "nf4_layer_error":
        L = q.lib()
        arr = (q.nf4_layer * 1)(_L())
        assert L.nf4_layer_error(arr, 1, f, None, FAKE, 1 << 20, None) == q.NF4_E_ARG
        assert L.nf4_layer_error(arr, 1, f, FAKE + 4, FAKE, 1 << 20, None) == q.NF4_E_ALIGN
        # absmax optional with double quant, required without
        assert _call(name, [_L(absmax=None)], q.fmt(dq=False)) == q.NF4_E_ARG
    if name in ("nf4_dequantize", "nf4_dequantize_masked"):
        assert _call(name, [_L(absmax=None)], q.fmt(dq=False)) == q.NF4_E_ARG
    if name == "nf4_dequantize_masked":
        assert _call(name, [_L()], f, skip=None) == q.NF4_E_ARG


@pytest.mark.parametrize("name", CODEC)
def test_tile_count_limit(name):
    """Fewer than 2^31 - 2^20 tiles of 16,384 weights per call (checked before
    anything is enqueued, so fake pointers suffice): 64 matrices of 2^39
    weights are 2^31 tiles; exactly at the limit is refused, one tile below
    it passes the size checks."""
    f = q.fmt()
    big = [_L(n=1 << 39) for _ in range(64)]
    assert _call(name, big, f) == q.NF4_E_UNSUPPORTED
    assert q.nf4_workspace_bytes([1 << 39] * 64, f) == 0
    limit = (1 << 31) - (1 << 20)                       # tiles
    at = [1 << 39] * 63 + [(limit - 63 * (1 << 25)) << 14]
    assert sum(n >> 14 for n in at) == limit
    assert _call(name, [_L(n=n) for n in at], f) == q.NF4_E_UNSUPPORTED
    assert q.nf4_workspace_bytes(at, f) == 0
    below = at[:-1] + [at[-1] - (1 << 14)]
    assert q.nf4_workspace_bytes(below, f) > 0


@pytest.mark.parametrize("name", CODEC)
def test_misaligned_pointers(name):
    f = q.fmt()
    fields = {"nf4_quantize": {"w": 16, "codes": 16, "absmax": 4, "scale2": 4},
              "nf4_double_quant": {"absmax": 4, "scale2": 4},
              "nf4_dequantize": {"codes": 16, "scale2": 4, "out": 16},
              "nf4_dequantize_masked": {"codes": 16, "scale2": 4, "out": 16},
              "nf4_layer_error": {"w": 16, "codes": 16, "absmax": 4, "scale2": 4}}[name]
    for field, a in fields.items():
        for off in (1, 2, 4, a // 2) if a > 2 else (1,):
            if off % a:
                assert _call(name, [_L(**{field: FAKE + off})], f) == q.NF4_E_ALIGN, (field, off)


@pytest.mark.parametrize("name", CODEC)
def test_workspace_checks(name):
    f = q.fmt()
    ns = [16384 * 5 + 3]
    tab_only = 256
    tiles = (ns[0] + 16383) // 16384
    rec = ((tiles * 8 + 255) // 256) * 256                       # 8-byte tile records
    part = ((tiles * 4 * 8 + 255) // 256) * 256                  # fp64 partials, 32 B per tile
    assert q.nf4_workspace_bytes(ns, f) == tab_only + rec + 2 * part
    # quantise: table + tile records; fused pass: + error partials; dequantisation: table +
    # a 32-byte record per tile; double quant: table only
    small = {"nf4_quantize": tab_only + rec, "nf4_double_quant": tab_only,
             "nf4_layer_error": tab_only + rec + part, "nf4_dequantize": tab_only + part,
             "nf4_dequantize_masked": tab_only + part}[name] - 1
    assert _call(name, [_L(n=ns[0])], f, ws=None) == q.NF4_E_WORKSPACE
    assert _call(name, [_L(n=ns[0])], f, ws=FAKE + 64) == q.NF4_E_WORKSPACE
    assert _call(name, [_L(n=ns[0])], f, ws_bytes=small) == q.NF4_E_WORKSPACE


def test_select_argument_errors():
    L = q.lib()
    ok = dict(err=FAKE, cost=FAKE, nl=10, budget=-1, kcap=-1, sel=FAKE, k=FAKE, ws=FAKE,
              wsb=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return L.aqlora_select_topk(a["err"], a["cost"], a["nl"], a["budget"], a["kcap"],
                                    a["sel"], a["k"], a["ws"], a["wsb"], None)
    for fld in ("err", "cost", "sel", "k"):
        assert call(**{fld: None}) == q.NF4_E_ARG
    assert call(nl=0) == q.NF4_E_ARG
    assert call(nl=65537) == q.NF4_E_ARG
    assert call(err=FAKE + 4) == q.NF4_E_ALIGN
    assert call(cost=FAKE + 4) == q.NF4_E_ALIGN
    assert call(k=FAKE + 2) == q.NF4_E_ALIGN
    assert call(ws=None) == q.NF4_E_WORKSPACE
    assert call(wsb=q.aqlora_workspace_bytes(10) - 1) == q.NF4_E_WORKSPACE


def test_status_strings():
    for s in range(6):
        assert q.lib().nf4_status_str(s)
    assert q.lib().nf4_status_str(99) == b"unknown status"


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful where no GPU exists")
def test_hip_failure_surfaces_as_status():
    """Valid arguments with no device: the first HIP call fails and the call
    reports NF4_E_HIP with the HIP code kept for nf4_last_hip_error()."""
    st = _call("nf4_quantize", [_L()], q.fmt())
    assert st == q.NF4_E_HIP
    assert q.lib().nf4_last_hip_error() != 0


def test_layer_error_norm_arguments():
    L = q.lib()
    f = q.fmt()
    ns = [16384 * 5 + 3]
    arr = (q.nf4_layer * 1)(_L(n=ns[0]))
    need = q.nf4_workspace_bytes(ns, f)
    ok = dict(err=FAKE, sq=FAKE + 1024, ws=FAKE, wsb=need)

    def call(**kw):
        a = dict(ok, **kw)
        return L.nf4_layer_error_norm(arr, 1, f, a["err"], a["sq"], a["ws"], a["wsb"], None)
    assert call(sq=None) == q.NF4_E_ARG
    assert call(err=None) == q.NF4_E_ARG
    assert call(sq=FAKE + 4) == q.NF4_E_ALIGN
    assert call(err=FAKE + 4) == q.NF4_E_ALIGN
    assert call(wsb=need - 1) == q.NF4_E_WORKSPACE      # needs both partial arrays
    assert L.nf4_layer_error_norm(arr, 0, f, FAKE, FAKE, FAKE, need, None) == q.NF4_E_ARG
    assert L.nf4_layer_error_norm(arr, 1, q.nf4_format(0, 32, 0), FAKE, FAKE, FAKE, need,
                                  None) == q.NF4_E_UNSUPPORTED


def test_select_variant_argument_errors():
    L = q.lib()
    nl = 10
    ge_ok = np.array([3, 7, 10], np.int32)
    ok = dict(err=FAKE, denom=None, cost=FAKE, nl=nl, ge=ge_ok, ng=3, budget=-1, kcap=-1,
              rule=0, sel=FAKE, k=FAKE, ws=FAKE, wsb=q.aqlora_workspace_bytes(nl))

    def call(**kw):
        a = dict(ok, **kw)
        ge = a["ge"]
        gp = None if ge is None else np.ascontiguousarray(ge, np.int32).ctypes.data
        return L.aqlora_select(a["err"], a["denom"], a["cost"], a["nl"], gp, a["ng"],
                               a["budget"], a["kcap"], a["rule"], a["sel"], a["k"], a["ws"],
                               a["wsb"], None)
    for fld in ("err", "cost", "sel", "k"):
        assert call(**{fld: None}) == q.NF4_E_ARG
    assert call(nl=0) == q.NF4_E_ARG
    assert call(nl=65537, ge=None) == q.NF4_E_ARG
    assert call(rule=2) == q.NF4_E_ARG
    assert call(rule=-1) == q.NF4_E_ARG
    assert call(ge=[3, 7, 9], ng=3) == q.NF4_E_ARG          # last != nl
    assert call(ge=[3, 3, 10], ng=3) == q.NF4_E_ARG         # not strictly increasing
    assert call(ge=[0, 5, 10], ng=3) == q.NF4_E_ARG         # empty first group
    assert call(ge=[3, 7, 10], ng=0) == q.NF4_E_ARG
    assert call(ge=np.arange(1, 12, dtype=np.int32), ng=11) == q.NF4_E_ARG   # ngroups > nl
    assert call(err=FAKE + 4) == q.NF4_E_ALIGN
    assert call(denom=FAKE + 4) == q.NF4_E_ALIGN
    assert call(cost=FAKE + 4) == q.NF4_E_ALIGN
    assert call(k=FAKE + 2) == q.NF4_E_ALIGN
    assert call(ws=None) == q.NF4_E_WORKSPACE
    assert call(wsb=q.aqlora_workspace_bytes(nl) - 1) == q.NF4_E_WORKSPACE


def test_matmul_arguments():
    L = q.lib()
    f = q.fmt()
    rows, cols = 256, 384

    def call(rows=rows, cols=cols, n=None, codes=FAKE, qa=FAKE, s2=FAKE, absmax=None, fmt=f,
             backward=0, x=FAKE, m=10, out=FAKE, out_fp32=1):
        lay = q.nf4_layer(rows * cols if n is None else n, None, codes, absmax, qa, s2, None)
        return L.nf4_matmul(ctypes.byref(lay), rows, cols, fmt, backward, x, m, out, out_fp32, None)
    assert call(fmt=q.nf4_format(2, 64, 256)) == q.NF4_E_UNSUPPORTED
    assert call(fmt=q.fmt(q.NF4_FP16, True), m=0) == q.NF4_E_ARG       # fp16 accepted
    assert call(fmt=q.nf4_format(0, 32, 256)) == q.NF4_E_UNSUPPORTED
    assert call(rows=200, n=200 * cols) == q.NF4_E_UNSUPPORTED
    assert call(cols=100, n=rows * 100) == q.NF4_E_UNSUPPORTED
    assert call(n=rows * cols - 1) == q.NF4_E_ARG
    assert call(m=0) == q.NF4_E_ARG
    assert call(m=1 << 31) == q.NF4_E_ARG
    assert call(backward=2) == q.NF4_E_ARG
    assert call(out_fp32=3) == q.NF4_E_ARG
    assert call(x=None) == q.NF4_E_ARG
    assert call(out=None) == q.NF4_E_ARG
    assert call(codes=None) == q.NF4_E_ARG
    assert call(qa=None) == q.NF4_E_ARG
    assert call(s2=None) == q.NF4_E_ARG
    assert call(fmt=q.fmt(dq=False), absmax=None) == q.NF4_E_ARG
    assert call(codes=FAKE + 4) == q.NF4_E_ALIGN
    assert call(x=FAKE + 8) == q.NF4_E_ALIGN
    assert call(out=FAKE + 8) == q.NF4_E_ALIGN
    assert call(s2=FAKE + 2) == q.NF4_E_ALIGN
    assert L.nf4_matmul(None, rows, cols, f, 0, FAKE, 10, FAKE, 1, None) == q.NF4_E_ARG


def test_matmul_split_workspace_and_arguments():
    """The split count depends on the shape only: the 14B FFN shape splits at
    small m and not at m = 4096; the workspace is parts x m x ncol fp32 (256-B
    rounded); a short or missing workspace is refused before anything is
    enqueued, and the other checks are nf4_matmul's."""
    L = q.lib()
    f = q.fmt()
    rows, cols = 13824, 5120
    for backward in (0, 1):
        ncol = cols if backward else rows
        w16 = q.nf4_matmul_workspace_bytes(rows, cols, backward, 16)
        assert w16 > 0 and w16 % 256 == 0 and w16 % (16 * ncol * 4) == 0
        parts = w16 // (16 * ncol * 4)
        assert 2 <= parts <= 16
    # m = 4096: 864 (forward) or 320 (backward) tiles of 256 x 256 on 256 CUs;
    # the 96 or 64 leftover tiles' reductions split 2 or 4 ways, one 256 x 256
    # fp32 block per (split, tile)
    assert q.nf4_matmul_workspace_bytes(rows, cols, 0, 4096) == 2 * 96 * 256 * 256 * 4
    assert q.nf4_matmul_workspace_bytes(rows, cols, 1, 4096) == 4 * 64 * 256 * 256 * 4
    # whole rounds only (4096 x 4096, m = 4096: 256 tiles): no workspace
    assert q.nf4_matmul_workspace_bytes(4096, 4096, 0, 4096) == 0
    # the parity test's shapes: 320 tiles (ragged rows, a 128-column tail), 4 splits
    # of 16 k-steps; 352 tiles, 2 splits of 16 k-steps
    assert q.nf4_matmul_workspace_bytes(4992, 4096, 0, 3900) == 4 * 64 * 256 * 256 * 4
    assert q.nf4_matmul_workspace_bytes(4096, 4992, 1, 3900) == 4 * 64 * 256 * 256 * 4
    assert q.nf4_matmul_workspace_bytes(5632, 2048, 0, 4096) == 2 * 96 * 256 * 256 * 4
    assert q.nf4_matmul_workspace_bytes(2048, 5632, 1, 4096) == 2 * 96 * 256 * 256 * 4
    # more than half a round left over (400 tiles: 144 left) or a reduction too
    # short to split (16 k-steps): none
    assert q.nf4_matmul_workspace_bytes(6400, 4096, 0, 4096) == 0
    assert q.nf4_matmul_workspace_bytes(4992, 1024, 0, 3900) == 0
    assert q.nf4_matmul_workspace_bytes(rows, cols, 0, 0) == 0
    assert q.nf4_matmul_workspace_bytes(200, cols, 0, 16) == 0
    assert L.nf4_matmul_workspace_bytes(rows, cols, 2, 16) == 0
    lay = q.nf4_layer(rows * cols, None, FAKE, None, FAKE, FAKE, None)
    need = q.nf4_matmul_workspace_bytes(rows, cols, 0, 16)

    def call(ws=FAKE, wsb=need, m=16, backward=0, x=FAKE, fmt=f):
        return L.nf4_matmul_ws(ctypes.byref(lay), rows, cols, fmt, backward, x, m, FAKE, 1, ws, wsb, None)
    assert call(wsb=need - 1) == q.NF4_E_WORKSPACE
    assert call(ws=None) == q.NF4_E_WORKSPACE
    assert call(ws=FAKE + 16) == q.NF4_E_WORKSPACE
    assert call(m=0) == q.NF4_E_ARG
    assert call(x=FAKE + 8) == q.NF4_E_ALIGN
    assert call(fmt=q.nf4_format(0, 32, 256)) == q.NF4_E_UNSUPPORTED


def test_few_token_forward_workspace():
    """Forward with m <= 32 takes the few-token kernel: parts of at most 8
    super-chunks of 128 k (4 above 16 tokens), sized for about 2,048 (16-row
    group, part) waves, so the workspace is ceil((cols/128) / sc) x m x rows
    fp32 with sc = clamp((cols/128) (rows/16) / 2048, 1, 8 or 4); m = 33 and
    backward keep the split reduction's count (at most 16 parts of whole
    k-steps)."""
    def expect(rows, cols, m):
        nsc, groups = cols // 128, rows // 16
        sc = min(8 if m <= 16 else 4, max(1, nsc * groups // 2048))
        parts = -(-nsc // sc)
        return -(-(parts * m * rows * 4) // 256) * 256
    for rows, cols in ((128, 128), (256, 384), (128, 1024), (8192, 1408), (13824, 5120),
                       (5120, 13824), (5120, 5120), (4096, 4096), (128, 65536)):
        for m in (1, 5, 16, 17, 32):
            assert q.nf4_matmul_workspace_bytes(rows, cols, False, m) == expect(rows, cols, m), (rows, cols, m)
        for m, bwd in ((33, False), (16, True)):
            w = q.nf4_matmul_workspace_bytes(rows, cols, bwd, m)
            ncol = cols if bwd else rows
            parts = w // (m * ncol * 4)
            assert w == 0 or (2 <= parts <= 16 and w == -(-(parts * m * ncol * 4) // 256) * 256), \
                (rows, cols, m, bwd)
    # one part of 1..8 super-chunks covers a 128-wide reduction or the 14B FFN's 5120
    assert q.nf4_matmul_workspace_bytes(128, 128, False, 16) == 16 * 128 * 4
    assert q.nf4_matmul_workspace_bytes(13824, 5120, False, 16) == 5 * 16 * 13824 * 4
    assert q.nf4_matmul_workspace_bytes(13824, 5120, False, 32) == 10 * 32 * 13824 * 4


def test_variant_helpers_and_arguments():
    for block in (32, 64, 128, 256):
        for kind in range(4):
            v = q.variant(q.NF4_BF16, block, kind)
            for n in (1, 31, 4097, 70_778_880):
                assert q.nf4_storage_bytes_variant(n, v) == oracle.storage_bytes_ex(n, block, kind)
    assert q.nf4_storage_bytes_variant(100, q.variant(block=48)) == -1
    assert q.nf4_storage_bytes_variant(100, q.variant(kind=4)) == -1
    L = q.lib()
    v = q.variant(q.NF4_BF16, 128, 3)
    ns = [128 * 256 * 2 + 5]
    need = q.nf4_workspace_bytes_variant(ns, v)
    groups = 3
    assert need == 256 + max(2 * (((groups * 8) + 255) // 256) * 256, ((groups * 64) + 255) // 256 * 256)

    def call(layer=None, vv=v, mean=FAKE, err=FAKE, ws=FAKE, wsb=need):
        arr = (q.nf4_layer * 1)(layer or _L(n=ns[0]))
        return L.nf4_layer_error_variant(arr, 1, vv, mean, err, ws, wsb, None)
    assert call(vv=q.variant(block=96)) == q.NF4_E_UNSUPPORTED
    assert call(vv=q.variant(kind=7)) == q.NF4_E_UNSUPPORTED
    assert call(mean=None) == q.NF4_E_ARG                        # kinds 2-3 write the mean
    assert call(err=None) == q.NF4_E_ARG
    assert call(layer=_L(n=ns[0], absmax=None)) == q.NF4_E_ARG    # absmax is always written
    assert call(layer=_L(n=ns[0], qabsmax=None)) == q.NF4_E_ARG
    assert call(mean=FAKE + 2) == q.NF4_E_ALIGN
    assert call(err=FAKE + 4) == q.NF4_E_ALIGN
    assert call(wsb=need - 1) == q.NF4_E_WORKSPACE
    arr = (q.nf4_layer * 1)(_L(n=ns[0]))
    assert L.nf4_dequantize_variant(arr, 1, v, None, FAKE, need, None) == q.NF4_E_ARG
    assert L.nf4_dequantize_variant(arr, 1, q.variant(block=12), FAKE, FAKE, need, None) == q.NF4_E_UNSUPPORTED


def test_noalloc_entry_checks_before_any_hip_call():
    """nf4_layer_error_noalloc: the same argument checks as nf4_layer_error,
    and a call whose table and partials exceed the fixed scratch is rejected
    with NF4_E_WORKSPACE on the host (stand-in pointers, nothing enqueued)."""
    L = q.lib()
    f = q.fmt()
    cap = q.nf4_noalloc_scratch_bytes()
    assert cap == 32 << 20

    def call(layers, f=f, err=FAKE):
        arr = (q.nf4_layer * max(1, len(layers)))(*layers)
        return L.nf4_layer_error_noalloc(arr, len(layers), f, err, None)

    assert call([_L()], err=None) == q.NF4_E_ARG
    assert call([]) == q.NF4_E_ARG
    assert call([_L(n=0)]) == q.NF4_E_ARG
    assert call([_L(w=FAKE + 2)]) == q.NF4_E_ALIGN
    assert call([_L()], err=FAKE + 4) == q.NF4_E_ALIGN
    assert call([_L()], f=q.nf4_format(0, 32, 0)) == q.NF4_E_UNSUPPORTED
    assert call([_L(qabsmax=None)]) == q.NF4_E_ARG
    # tiles of 16,384 weights, 32 B of partials each, after the 256-byte table
    tiles_max = (cap - 512) // 40
    assert call([_L(n=(tiles_max + 1) * 16384)]) == q.NF4_E_WORKSPACE
    assert call([_L(n=1 << 35)]) == q.NF4_E_WORKSPACE
