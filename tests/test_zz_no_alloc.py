"""nf4_layer_error_noalloc (the fused pass in the library's fixed per-device
scratch, for callers that cannot allocate) against nf4_layer_error with a
caller workspace: every output bitwise equal, on two calls in a row, the
second with a smaller input, in bf16 with double quant and fp16 without.
The workspace entry point is itself checked bit for bit against the oracle
in the parity tests; here the smaller calls are also checked against the
oracle directly."""
import numpy as np
import pytest
import torch

import oracle
import quantized_lora_fine_nf4_amd as q
import synth
from conftest import print_case
from gpu_util import compare_layer, layerset, rel_err

pytestmark = pytest.mark.gpu

TILE = 16384


def _stack(sizes, dtype, seed):
    return [synth.generate_raw(seed + i, n, dtype=dtype, sigma=0.02, outlier_frac=0.001)
            for i, n in enumerate(sizes)]


def _outputs(ls, f):
    out = {"codes": ls.codes.cpu().numpy()}
    if ls.absmax is not None:
        out["absmax"] = ls.absmax.cpu().numpy().view(np.uint32)
    if f.dq_group:
        out["qabsmax"] = ls.qabsmax.cpu().numpy()
        out["scale2"] = ls.scale2.cpu().numpy().view(np.uint32)
    return out


@pytest.mark.parametrize("dtype,dq", [(q.NF4_BF16, True), (q.NF4_FP16, False)])
def test_noalloc_equals_workspace_entry(dtype, dq):
    f = q.fmt(dtype, dq)
    calls = [
        # first call: several whole and ragged tiles per matrix, odd n, a
        # matrix smaller than one block
        [5 * TILE + 777, 3 * TILE, 100_003, 4096 * 1024 + 1, 63, 2 * TILE + 64],
        # second call, smaller: fewer matrices and tiles than the first left
        # in the scratch
        [TILE + 1, 999, 65],
    ]
    for step, sizes in enumerate(calls):
        print_case("noalloc", "dtype", dtype, "dq", dq, "call", step, "sizes", sizes)
        ws_host = _stack(sizes, dtype, 9100 + 50 * step + 10 * dtype)
        ref_ls = layerset(ws_host, f)
        ws = torch.empty(q.nf4_workspace_bytes(ref_ls.ns, f), dtype=torch.uint8, device="cuda")
        err_ref = torch.full((len(sizes),), float("nan"), dtype=torch.float64, device="cuda")
        q.nf4_layer_error(ref_ls, f, err_ref, ws)
        ls = layerset(ws_host, f)
        err = torch.full((len(sizes),), float("nan"), dtype=torch.float64, device="cuda")
        q.nf4_layer_error_noalloc(ls, f, err)
        torch.cuda.synchronize()
        assert torch.equal(err.view(torch.int64), err_ref.view(torch.int64)), (step, err, err_ref)
        a, b = _outputs(ls, f), _outputs(ref_ls, f)
        for k in a:
            assert np.array_equal(a[k], b[k]), (step, k)
        if step == 1:
            errs = err.cpu().numpy()
            for i, w in enumerate(ws_host):
                ref = compare_layer(ls, i, w, dtype, dq)
                assert rel_err(errs[i], ref["err"]) <= 1e-5, (i, errs[i], ref["err"])

