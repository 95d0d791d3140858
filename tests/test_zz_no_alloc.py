"""The DGrad entry point that allocates nothing (fp8_gemm_dgrad_split_noalloc):
called through the C ABI, it must give the workspace-taking
fp8_gemm_dgrad_split's output bit for bit (same kernels, same partition),
on two calls in a row, the second with a smaller input, so the second reuses
the library's scratch array with the first call's partial sums still in it;
and where no split applies it must be the plain DGrad."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_02_amd as fb
import oracle
from gpu_util import TOL, banner, dev_strided, host

pytestmark = pytest.mark.gpu


def _inputs(N, D, C, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    dY = (rng.standard_normal((N, D)) * np.exp(rng.uniform(-4, 2, (1, D)))).astype(np.float32)
    return W, dY


def _with_workspace(gq, gs, wqT, ws, N, D, C, out_dtype):
    """The existing entry point with a caller-owned workspace from torch."""
    dx = fb._new_out(N, C, out_dtype, gq.device).fill_(float("nan"))
    nbytes = fb.lib().fp8_gemm_dgrad_split_bytes(N, D, C)
    work = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device="cuda")
    fb._call("fp8_gemm_dgrad_split", fb._ptr(gq), fb._ld(gq), fb._ptr(gs), fb._ld(gs), fb._ptr(wqT),
             fb._ld(wqT), fb._ptr(ws), fb._ld(ws), fb._ptr(dx), fb._out_dtype_code(out_dtype), fb._ld(dx),
             N, D, C, fb._ptr(work), nbytes, fb._stream(gq.device))
    return dx


def _no_alloc(gq, gs, wqT, ws, N, D, C, out_dtype):
    dx = fb._new_out(N, C, out_dtype, gq.device).fill_(float("nan"))
    fb._call("fp8_gemm_dgrad_split_noalloc", fb._ptr(gq), fb._ld(gq), fb._ptr(gs), fb._ld(gs), fb._ptr(wqT),
             fb._ld(wqT), fb._ptr(ws), fb._ld(ws), fb._ptr(dx), fb._out_dtype_code(out_dtype), fb._ld(dx),
             N, D, C, fb._stream(gq.device))
    return dx


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_no_alloc_dgrad_equals_workspace_dgrad(out_dtype):
    # first the decode-shaped DGrad (64 x 4096, K = 24576: 8 ranges, the
    # full 8 MiB of scratch), then a smaller ragged one (2 ranges) that
    # reads back a scratch array still holding the first call's sums
    for N, D, C, seed in ((64, 24576, 4096, 1), (37, 2304, 301, 2)):
        banner(f"no-alloc dgrad N={N} D={D} C={C} {out_dtype}")
        assert fb.lib().fp8_gemm_dgrad_split_bytes(N, D, C) > 0
        W, dY = _inputs(N, D, C, seed)
        gq, gs = fb.fp8_quantize_act_1x128(dev_strided(dY))
        wq, ws, wqT = fb.fp8_quantize_weight_128x128(dev_strided(W))
        got = _no_alloc(gq, gs, wqT, ws, N, D, C, out_dtype)
        want = _with_workspace(gq, gs, wqT, ws, N, D, C, out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (N, D, C)
        ogq, ogs = oracle.quant_1x128(dY)
        owq, ows, _ = oracle.quant_128x128(W, with_transpose=False)
        err = oracle.rel_row_error(host(got), oracle.dgrad(ogq, ogs, owq, ows, D, C))
        banner(f"no-alloc dgrad rel row error {err:.3e}")
        assert err <= TOL


def test_no_alloc_dgrad_without_split_is_plain_dgrad():
    N, D, C = 65, 4096, 512                       # more than 64 rows: no split, no scratch
    assert fb.lib().fp8_gemm_dgrad_split_bytes(N, D, C) == 0
    W, dY = _inputs(N, D, C, 3)
    gq, gs = fb.fp8_quantize_act_1x128(dev_strided(dY))
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(dev_strided(W))
    got = _no_alloc(gq, gs, wqT, ws, N, D, C, torch.float32)
    want = fb.fp8_gemm_dgrad(gq, gs, wqT, ws, N, D, C, out_dtype=torch.float32)
    assert torch.equal(got, want)


def test_no_alloc_dgrad_rejects_bad_arguments_before_any_launch():
    N, D, C = 64, 4096, 512
    W, dY = _inputs(N, D, C, 4)
    gq, gs = fb.fp8_quantize_act_1x128(dev_strided(dY))
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(dev_strided(W))
    dx = fb._new_out(N, C, torch.float32, gq.device).zero_()
    L = fb.lib()
    st = fb._stream(gq.device)
    # null output, then a leading dimension below the row length
    assert L.fp8_gemm_dgrad_split_noalloc(fb._ptr(gq), fb._ld(gq), fb._ptr(gs), fb._ld(gs), fb._ptr(wqT),
                                          fb._ld(wqT), fb._ptr(ws), fb._ld(ws), None, 0, C, N, D, C, st) == 1
    assert L.fp8_gemm_dgrad_split_noalloc(fb._ptr(gq), fb._ld(gq), fb._ptr(gs), fb._ld(gs), fb._ptr(wqT),
                                          fb._ld(wqT), fb._ptr(ws), fb._ld(ws), fb._ptr(dx), 0, C - 4,
                                          N, D, C, st) == 2
    torch.cuda.synchronize()
    assert torch.all(dx == 0)
