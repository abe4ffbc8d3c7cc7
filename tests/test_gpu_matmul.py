"""GPU parity of the fused NF4 matmul (nf4_matmul) against the oracle.

The weight's NF4 form is made by the oracle on the host and uploaded, so the
test isolates the matmul.  Reference: the oracle's dequantised weight and an
fp64 product.  Bound (fp32 accumulation of exact bf16 or fp16 products over K
terms): |out - ref| <= 2 K 2^-24 (|x| |W|^T) elementwise.  The 16-bit output
equals the round-to-nearest-even of the same kernel's fp32 output.  bf16 and
fp16, ragged m (1, 77, 300), several tile counts, double quant on and off,
forward and backward; a shape whose last tiles run as halves, every element;
the 14B stack's FFN shape (13824 x 5120) at m = 4096 on sampled rows.  The split-reduction path (nf4_matmul_ws) on shapes it
splits, against the same bound, deterministic, and the FFN shape at m = 16
and 32; its split of the tiles left over after whole rounds (two shapes, and
the FFN shape at m = 4096); its few-token forward kernel (m <= 32: 1, 5, 16, 17, 32) the same way.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_lora_fine_nf4_amd as q
import synth
from conftest import print_case

pytestmark = pytest.mark.gpu
BF16, FP16 = q.NF4_BF16, q.NF4_FP16
TORCH16 = {BF16: torch.bfloat16, FP16: torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    q.lib()
    yield
    torch.cuda.synchronize()


class DevWeight:
    """A matrix's NF4 form (from the oracle) in device memory."""

    def __init__(self, rows, cols, seed, dq, outliers=0.0, dtype=BF16):
        w = synth.generate_raw(seed, rows * cols, dtype=dtype, outlier_frac=outliers)
        codes, absmax = oracle.quantize(w, dtype)
        self.consts = dict(absmax=absmax)
        self.codes = torch.from_numpy(codes).cuda()
        self.absmax = torch.from_numpy(absmax).cuda()
        self.q = self.s2 = None
        if dq:
            qa, s2 = oracle.double_quant(absmax)
            self.consts = dict(qabsmax=qa, scale2=s2)
            self.q = torch.from_numpy(qa).cuda()
            self.s2 = torch.from_numpy(s2).cuda()
        self.np_codes = codes
        self.rows, self.cols, self.dq, self.dtype = rows, cols, dq, dtype
        ptr = lambda t: None if t is None else int(t.data_ptr())
        self.layer = q.nf4_layer(rows * cols, None, ptr(self.codes),
                                 None if dq else ptr(self.absmax), ptr(self.q), ptr(self.s2), None)

    def dense(self):
        y = oracle.dequantize(self.np_codes, self.rows * self.cols, self.dtype, **self.consts)
        return oracle.from16(y, self.dtype).astype(np.float64).reshape(self.rows, self.cols)


def _x(m, k, seed, dtype=BF16):
    rng = np.random.default_rng(seed)
    return oracle.to16_rne(rng.standard_normal(m * k).astype(np.float32), dtype).reshape(m, k)


def _run(W, xb, backward, out_f32=True):
    m = xb.shape[0]
    ncol = W.cols if backward else W.rows
    x = torch.from_numpy(xb.view(np.int16)).cuda()
    out = torch.full((m, ncol), float("nan"), dtype=torch.float32 if out_f32 else TORCH16[W.dtype],
                     device="cuda")
    q.nf4_matmul(W.layer, W.rows, W.cols, q.fmt(W.dtype, W.dq), x, out, backward=backward)
    torch.cuda.synchronize()
    return out


def _check(out, xb, W, backward, rows_idx=None):
    x = oracle.from16(xb, W.dtype).astype(np.float64).reshape(xb.shape)
    if rows_idx is not None:
        x = x[rows_idx]
    Wd = W.dense()
    ref = x @ Wd if backward else x @ Wd.T
    mag = np.abs(x) @ np.abs(Wd) if backward else np.abs(x) @ np.abs(Wd).T
    K = W.rows if backward else W.cols
    got = out.double().cpu().numpy()
    if rows_idx is not None:
        got = got[rows_idx]
    assert np.all(np.isfinite(got))
    bound = 2.0 * K * 2.0 ** -24 * mag + 1e-30
    excess = np.abs(got - ref) / bound
    worst = float(excess.max())
    assert worst <= 1.0, (worst, np.unravel_index(int(excess.argmax()), excess.shape))
    return worst


@pytest.mark.parametrize("backward", [False, True], ids=["fwd", "bwd"])
@pytest.mark.parametrize("dq", [False, True], ids=["nodq", "dq"])
@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 256)], ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("m", [1, 77, 128, 300])
@pytest.mark.parametrize("dtype", [BF16, FP16], ids=["bf16", "fp16"])
def test_matmul_matches_oracle(dtype, m, shape, dq, backward):
    rows, cols = shape
    print_case("nf4_matmul", dtype, m, rows, cols, "dq" if dq else "nodq", "bwd" if backward else "fwd")
    W = DevWeight(rows, cols, 7000 + rows + cols, dq, outliers=0.002, dtype=dtype)
    xb = _x(m, rows if backward else cols, 11 * m + rows, dtype)
    out = _run(W, xb, backward)
    _check(out, xb, W, backward)
    # 16-bit output: RNE of the same fp32 sums
    o16 = _run(W, xb, backward, out_f32=False)
    assert torch.equal(o16, out.to(TORCH16[dtype]))


def test_matmul_is_deterministic():
    W = DevWeight(256, 256, 42, True)
    xb = _x(300, 256, 43)
    a = _run(W, xb, False)
    b = _run(W, xb, False)
    assert torch.equal(a, b)


@pytest.mark.slow
@pytest.mark.parametrize("backward,dtype", [(False, BF16), (True, BF16), (False, FP16), (True, FP16)],
                         ids=["fwd-bf16", "bwd-bf16", "fwd-fp16", "bwd-fp16"])
def test_matmul_fullsize_ffn_sampled(backward, dtype):
    rows, cols, m = 13824, 5120, 4096
    print_case("nf4_matmul full size", dtype, rows, cols, m, "bwd" if backward else "fwd")
    W = DevWeight(rows, cols, 99, True, outliers=0.0005, dtype=dtype)
    xb = _x(m, rows if backward else cols, 100, dtype)
    out = _run(W, xb, backward)
    rng = np.random.default_rng(5)
    idx = np.sort(np.r_[0, m - 1, rng.integers(0, m, 6)])
    worst = _check(out, xb, W, backward, rows_idx=idx)
    print(f"[{'bwd' if backward else 'fwd'}] worst error / bound {worst:.3f}", flush=True)


@pytest.mark.parametrize("dq", [True, False], ids=["dq", "nodq"])
@pytest.mark.parametrize("m", [3300, 3100])
@pytest.mark.parametrize("backward", [False, True], ids=["fwd", "bwd"])
def test_matmul_tail_halves_match_oracle(backward, m, dq):
    """260 output tiles of 256 x 256 on 256 CUs: the 4 tiles past the whole
    round run in row pieces (128-row halves forward, 64-row quarters
    backward), some of them over the ragged last 228 or 28 rows and, at
    m = 3100, some entirely past the last row; every output element is
    checked, with double quant and with fp32 absmax."""
    rows, cols = (256, 5120) if backward else (5120, 256)
    print_case("nf4_matmul tail halves", m, rows, cols, "dq" if dq else "nodq", "bwd" if backward else "fwd")
    W = DevWeight(rows, cols, 515, dq, outliers=0.001)
    xb = _x(m, rows if backward else cols, 516)
    out = _run(W, xb, backward)
    _check(out, xb, W, backward)
    o16 = _run(W, xb, backward, out_f32=False)
    assert torch.equal(o16, out.to(torch.bfloat16))


def _run_ws(W, xb, backward, out_f32=True):
    m = xb.shape[0]
    ncol = W.cols if backward else W.rows
    x = torch.from_numpy(xb.view(np.int16)).cuda()
    out = torch.full((m, ncol), float("nan"), dtype=torch.float32 if out_f32 else TORCH16[W.dtype],
                     device="cuda")
    need = q.nf4_matmul_workspace_bytes(W.rows, W.cols, backward, m)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda") if need else None
    if ws is not None:
        ws.fill_(0xFF)   # stale NaN partials must not leak into the result
    q.nf4_matmul_ws(W.layer, W.rows, W.cols, q.fmt(W.dtype, W.dq), x, out, ws, backward=backward)
    torch.cuda.synchronize()
    return out, need


@pytest.mark.parametrize("backward", [False, True], ids=["fwd", "bwd"])
@pytest.mark.parametrize("dtype", [BF16, FP16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("m", [1, 77, 300])
def test_split_reduction_matches_oracle(m, dtype, backward):
    """nf4_matmul_ws on shapes it splits (few output tiles): within the same
    fp32 bound of the oracle's product, 16-bit output = RNE of its own fp32
    result, and bitwise equal from run to run."""
    rows, cols = 256, 384
    print_case("nf4_matmul_ws", dtype, m, rows, cols, "bwd" if backward else "fwd")
    W = DevWeight(rows, cols, 8100 + m, True, outliers=0.002, dtype=dtype)
    xb = _x(m, rows if backward else cols, 13 * m + 1, dtype)
    out, need = _run_ws(W, xb, backward)
    assert need > 0
    _check(out, xb, W, backward)
    again, _ = _run_ws(W, xb, backward)
    assert torch.equal(out, again)
    o16, _ = _run_ws(W, xb, backward, out_f32=False)
    assert torch.equal(o16, out.to(TORCH16[dtype]))


@pytest.mark.parametrize("m", [200, 300])
@pytest.mark.parametrize("dtype", [BF16, FP16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("backward", [False, True], ids=["fwd", "bwd"])
def test_split_large_tiles_matches_oracle(backward, dtype, m):
    """nf4_matmul_ws with more than 128 rows of x and a long reduction over
    few 256 x 256 tiles: the reduction is split across workgroups of the
    large-tile kernels (4 splits of 16 k-steps here).  The same bound,
    bitwise equal from run to run, stale workspace unused, and within the
    bound too through nf4_matmul, which takes the call unsplit."""
    rows, cols = (4096, 512) if backward else (512, 4096)
    ncol = cols if backward else rows
    print_case("nf4_matmul_ws large tiles split", dtype, m, rows, cols, "bwd" if backward else "fwd")
    W = DevWeight(rows, cols, 8700 + m + int(backward), True, outliers=0.002, dtype=dtype)
    xb = _x(m, rows if backward else cols, 19 * m + 3, dtype)
    out, need = _run_ws(W, xb, backward)
    assert need == 4 * m * ncol * 4
    _check(out, xb, W, backward)
    again, _ = _run_ws(W, xb, backward)
    assert torch.equal(out, again)
    o16, _ = _run_ws(W, xb, backward, out_f32=False)
    assert torch.equal(o16, out.to(TORCH16[dtype]))
    _check(_run(W, xb, backward), xb, W, backward)


@pytest.mark.parametrize("case,dtype,dq", [((3900, 4992, 4096, 4), BF16, True),
                                           ((4096, 5632, 2048, 2), BF16, True),
                                           ((3900, 4992, 4096, 4), FP16, False)],
                         ids=["320tiles-4splits", "352tiles-2splits", "320tiles-fp16-nodq"])
@pytest.mark.parametrize("backward", [False, True], ids=["fwd", "bwd"])
def test_tail_split_matches_oracle(backward, case, dtype, dq):
    """nf4_matmul_ws where the 256 x 256 tiles fill whole rounds and leave
    fewer than half a round over: the whole tiles run unsplit, the leftover
    tiles' reductions split (4 ways over 64 tiles, 2 ways over 96) into one
    fp32 block per (split, tile), added in split order.  The first shape has a
    ragged last row tile (60 rows) and a 128-column last column tile, both
    among the leftover tiles; it runs in bf16 with double quant and in fp16
    with fp32 absmax.  Checked on every row of the last four row tiles
    (which hold all the leftover tiles and some whole ones) and sampled rows
    above: the same fp32 bound, 16-bit output = RNE of its fp32 output,
    bitwise equal from run to run, stale workspace unused."""
    m, ncol, kred, splits = case
    rows, cols = (kred, ncol) if backward else (ncol, kred)
    print_case("nf4_matmul_ws tail split", m, rows, cols, dtype, "dq" if dq else "nodq",
               "bwd" if backward else "fwd")
    W = DevWeight(rows, cols, 8900 + m + int(backward), dq, outliers=0.001, dtype=dtype)
    xb = _x(m, kred, 23 * m + int(backward), dtype)
    out, need = _run_ws(W, xb, backward)
    tiles = -(-m // 256) * -(-ncol // 256)
    assert need == splits * (tiles - 256) * 256 * 256 * 4
    rng = np.random.default_rng(m)
    idx = np.unique(np.r_[np.arange(3072, m), 0, 255, 256, rng.integers(0, 3072, 8)])
    _check(out, xb, W, backward, rows_idx=idx)
    again, _ = _run_ws(W, xb, backward)
    assert torch.equal(out, again)
    o16, _ = _run_ws(W, xb, backward, out_f32=False)
    assert torch.equal(o16, out.to(TORCH16[dtype]))


# parts of 1 super-chunk (3 and 8 parts), 2 super-chunks with a last part of 1
# (6 parts), and 2 super-chunks in 10 parts over 68 workgroups of 64 rows
@pytest.mark.parametrize("shape", [(256, 384), (128, 1024), (8192, 1408), (4352, 2560)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("dq", [False, True], ids=["nodq", "dq"])
@pytest.mark.parametrize("dtype", [BF16, FP16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("m", [1, 5, 16, 17, 32])
def test_few_token_forward_matches_oracle(m, dtype, dq, shape):
    """nf4_matmul_ws forward with at most 32 tokens (one wave per 16 weight
    rows and one or two 16-row blocks of x, the reduction in parts): the same
    bound, 16-bit output = RNE of its fp32 output, bitwise equal from run to
    run, and stale workspace unused."""
    rows, cols = shape
    print_case("nf4_matmul_ws few tokens", dtype, m, rows, cols, "dq" if dq else "nodq")
    W = DevWeight(rows, cols, 8300 + m + rows, dq, outliers=0.002, dtype=dtype)
    xb = _x(m, cols, 17 * m + rows, dtype)
    out, need = _run_ws(W, xb, False)
    assert need > 0 and need % 256 == 0
    _check(out, xb, W, False)
    again, _ = _run_ws(W, xb, False)
    assert torch.equal(out, again)
    o16, _ = _run_ws(W, xb, False, out_f32=False)
    assert torch.equal(o16, out.to(TORCH16[dtype]))


def test_split_path_not_taken_equals_nf4_matmul():
    """A shape whose output tiles fill the GPU needs no workspace, and then
    nf4_matmul_ws is nf4_matmul bit for bit."""
    W = DevWeight(4096, 128, 77, True)
    xb = _x(2048, 128, 78)
    out, need = _run_ws(W, xb, False)
    assert need == 0
    assert torch.equal(out, _run(W, xb, False))


@pytest.mark.slow
@pytest.mark.parametrize("m", [512, 1536, 4096])
@pytest.mark.parametrize("backward", [False, True], ids=["fwd", "bwd"])
def test_split_fullsize_ffn_mid_m(backward, m):
    """The FFN weight at m = 512 and 1536 through nf4_matmul_ws (the
    large-tile kernels with the reduction split where planned), and at
    m = 4096 (whole rounds unsplit, the leftover tiles split), on sampled
    rows."""
    rows, cols = 13824, 5120
    print_case("nf4_matmul_ws full size mid m", rows, cols, m, "bwd" if backward else "fwd")
    W = DevWeight(rows, cols, 103, True, outliers=0.0005)
    xb = _x(m, rows if backward else cols, 104)
    out, need = _run_ws(W, xb, backward)
    rng = np.random.default_rng(7)
    # at m = 4096 the leftover tiles hold rows 3072 .. 4095
    idx = np.unique(np.r_[0, m - 1, rng.integers(0, m, 6), rng.integers(max(0, m - 1024), m, 4)])
    worst = _check(out, xb, W, backward, rows_idx=idx)
    print(f"[{'bwd' if backward else 'fwd'} m={m}] worst error / bound {worst:.3f}, workspace {need} B", flush=True)


@pytest.mark.slow
@pytest.mark.parametrize("m", [16, 32])
@pytest.mark.parametrize("backward", [False, True], ids=["fwd", "bwd"])
def test_split_fullsize_ffn_small_m(backward, m):
    rows, cols = 13824, 5120
    print_case("nf4_matmul_ws full size", rows, cols, m, "bwd" if backward else "fwd")
    W = DevWeight(rows, cols, 101, True, outliers=0.0005)
    xb = _x(m, rows if backward else cols, 102)
    out, need = _run_ws(W, xb, backward)
    assert need > 0
    worst = _check(out, xb, W, backward)
    print(f"[{'bwd' if backward else 'fwd'} m={m}] worst error / bound {worst:.3f}", flush=True)
