"""GPU parity of the dequantized-backward mode: the bf16 dequantization of
FP8 operands bit for bit against the oracle (1x128 row groups, 128x128
blocks, MX 1x32), the transposed operand copies the bf16 GEMM reads (bit
for bit), and the bf16 DGrad/WGrad GEMMs on those operands against the
oracle's binary64 product of the same bf16 values (2e-3 of the row norm:
bf16 output rounding plus fp32 accumulation)."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_02_amd as fb
import oracle
from block_scaled_fp8_02_amd import workloads as wl
from gpu_util import TOL, assert_bytes_equal, banner, dev, dev_strided, host

pytestmark = pytest.mark.gpu


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def rand_x(rng, shape, spread=10.0):
    return (rng.standard_normal(shape) * np.exp(rng.uniform(-spread, spread, (shape[0], 1)))).astype(np.float32)


@pytest.mark.parametrize("shape", [(1, 1), (3, 300), (129, 257), (300, 5), (256, 512)])
def test_dequantize_all_layouts(shape):
    banner(f"dequantize {shape}")
    rows, cols = shape
    rng = np.random.default_rng(rows * 7 + cols)
    x = rand_x(rng, shape)
    q, s = oracle.quant_1x128(x)
    got = bits_of(fb.fp8_dequantize_bf16(dev(q), dev_strided(s), fb.FP8B_SCALE_ROWS_1X128, cols))
    assert_bytes_equal(got, oracle.dequant_bf16_rows(q, s, cols), "1x128 rows")
    wq, ws, _ = oracle.quant_128x128(x, with_transpose=False)
    got = bits_of(fb.fp8_dequantize_bf16(dev(wq), dev(ws), fb.FP8B_SCALE_BLOCKS_128X128, cols))
    assert_bytes_equal(got, oracle.dequant_bf16_128x128(wq, ws, rows, cols), "128x128 blocks")
    mq, me = oracle.mx_quant_rows(x)
    got = bits_of(fb.fp8_dequantize_bf16(dev(mq), dev(me), fb.FP8B_SCALE_MX_1X32, cols))
    assert_bytes_equal(got, oracle.dequant_bf16_mx(mq, me, cols), "MX 1x32")


def test_dequantize_every_code_and_extreme_scales():
    banner("dequantize code classes")
    rng = np.random.default_rng(70)
    codes = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)
    q = codes[(np.arange(254)[:, None] + np.arange(256)[None, :]) % 254].astype(np.uint8)
    s = np.empty((254, 2), np.float32)
    s[:, 0] = np.ldexp(1.0, rng.integers(-140, 100, 254)).astype(np.float32)
    s[:, 1] = (rng.uniform(0.5, 2.0, 254) * np.exp(rng.uniform(-80, 80, 254))).astype(np.float32)
    got = bits_of(fb.fp8_dequantize_bf16(dev(q), dev(s), fb.FP8B_SCALE_ROWS_1X128, 256))
    assert_bytes_equal(got, oracle.dequant_bf16_rows(q, s, 256), "code classes")


@pytest.mark.parametrize("N,D,C", [(256, 384, 512), (200, 300, 260), (3, 130, 300)])
def test_dequant_backward_gemms(N, D, C):
    banner(f"dequantized backward N={N} D={D} C={C}")
    rng = np.random.default_rng(N + D + C + 71)
    X = oracle.bf16_rne(rng.standard_normal((N, C)).astype(np.float32))
    W = oracle.bf16_rne((rng.standard_normal((D, C)) * 0.02).astype(np.float32))
    dY = oracle.bf16_rne((rng.standard_normal((N, D)) * 1e-3).astype(np.float32))
    xq, xs = oracle.quant_1x128(X)
    wq, ws, _ = oracle.quant_128x128(W, with_transpose=False)
    dYd = dev_strided(dY)
    dx = host(fb.fp8_dequant_gemm_dgrad(dYd, dev(wq), dev(ws), fb.FP8B_SCALE_BLOCKS_128X128, N, D, C))
    want_dx = oracle.bf16_matmul(dY, oracle.dequant_bf16_128x128(wq, ws, D, C))
    e = oracle.rel_row_error(dx, want_dx)
    banner(f"  dgrad (128x128 W^) {e:.3e}")
    assert e <= TOL
    for out_dtype, beta in ((torch.bfloat16, 0), (torch.float32, 0), (torch.float32, 1)):
        dw0 = torch.full((D, C), 0.25, dtype=torch.float32, device="cuda") if beta else None
        dw = host(fb.fp8_dequant_gemm_wgrad(dYd, dev(xq), dev(xs), fb.FP8B_SCALE_ROWS_1X128, N, D, C,
                                            dw=dw0, out_dtype=out_dtype, beta=beta))
        want = oracle.bf16_matmul(np.ascontiguousarray(dY.T), oracle.dequant_bf16_rows(xq, xs, C))
        if beta:
            want = want + 0.25
        e = oracle.rel_row_error(dw, want)
        banner(f"  wgrad (1x128 X^) {out_dtype} beta {beta}: {e:.3e}")
        assert e <= (TOL if out_dtype == torch.bfloat16 else 1e-5)
    # MX forward operands
    mxq, mxe = oracle.mx_quant_rows(X)
    mwq, mwe = oracle.mx_quant_rows(W)
    dx = host(fb.fp8_dequant_gemm_dgrad(dYd, dev(mwq), dev(mwe), fb.FP8B_SCALE_MX_1X32, N, D, C))
    e = oracle.rel_row_error(dx, oracle.bf16_matmul(dY, oracle.dequant_bf16_mx(mwq, mwe, C)))
    banner(f"  dgrad (MX W^) {e:.3e}")
    assert e <= TOL
    dw = host(fb.fp8_dequant_gemm_wgrad(dYd, dev(mxq), dev(mxe), fb.FP8B_SCALE_MX_1X32, N, D, C))
    e = oracle.rel_row_error(dw, oracle.bf16_matmul(np.ascontiguousarray(dY.T), oracle.dequant_bf16_mx(mxq, mxe, C)))
    banner(f"  wgrad (MX X^) {e:.3e}")
    assert e <= TOL


def tile_rows(n: int, seed: int, tile: int = 256) -> np.ndarray:
    """One seeded row from every 256-row output tile, plus the first and last
    row: every 256 x 256 tile of the output has a checked row."""
    rng = np.random.default_rng(seed)
    r = [t + int(rng.integers(0, min(tile, n - t))) for t in range(0, n, tile)] + [0, n - 1]
    return np.unique(np.array(r, dtype=np.int64))


@pytest.mark.parametrize("N,D,C", [(200, 300, 260), (3, 130, 300), (256, 384, 512)])
def test_transposed_operand_copies(N, D, C):
    """The workspaces the bf16 GEMMs read, bit for bit: W^ transposed (DGrad),
    X^ transposed then dY transposed (WGrad), with columns [K, round_up(K,
    8)) of each workspace row written zero."""
    banner(f"transposed operand copies N={N} D={D} C={C}")
    rng = np.random.default_rng(N + 3 * D + C)
    X = oracle.bf16_rne(rand_x(rng, (N, C), 4.0))
    W = oracle.bf16_rne((rng.standard_normal((D, C)) * 0.02).astype(np.float32))
    dY = oracle.bf16_rne((rng.standard_normal((N, D)) * 1e-3).astype(np.float32))
    dYd = dev_strided(dY)
    bq, bs, _ = oracle.quant_128x128(W, with_transpose=False)
    mq, me = oracle.mx_quant_rows(W)
    for wq, ws, kind, deq in ((bq, bs, fb.FP8B_SCALE_BLOCKS_128X128, oracle.dequant_bf16_128x128(bq, bs, D, C)),
                              (mq, me, fb.FP8B_SCALE_MX_1X32, oracle.dequant_bf16_mx(mq, me, C))):
        work = fb._new_out(C, D, torch.bfloat16, dYd.device).fill_(float("nan"))
        fb.fp8_dequant_gemm_dgrad(dYd, dev(wq), dev(ws), kind, N, D, C, work=work)
        assert_bytes_equal(bits_of(work), np.ascontiguousarray(deq.T), f"W^T kind {kind}")
    aq, as_ = oracle.quant_1x128(X)
    nq, ne = oracle.mx_quant_rows(X)
    for xq, xs, kind, deq in ((aq, as_, fb.FP8B_SCALE_ROWS_1X128, oracle.dequant_bf16_rows(aq, as_, C)),
                              (nq, ne, fb.FP8B_SCALE_MX_1X32, oracle.dequant_bf16_mx(nq, ne, C))):
        work = fb._new_out(C + D, N, torch.bfloat16, dYd.device).fill_(float("nan"))
        fb.fp8_dequant_gemm_wgrad(dYd, dev(xq), dev(xs), kind, N, D, C, work=work)
        full = work.as_strided((C + D, (N + 7) // 8 * 8), work.stride())
        got = bits_of(full)
        assert_bytes_equal(got[:C, :N], np.ascontiguousarray(deq.T), f"X^T kind {kind}")
        assert_bytes_equal(got[C:, :N], np.ascontiguousarray(dY.T), "dY^T")
        assert np.all(got[:, N:] == 0), "pad columns of the workspace rows"


@pytest.mark.parametrize("N,D,C", [(37, 130, 200), (64, 1000, 136), (300, 77, 520)])
def test_dequant_backward_ignores_row_padding(N, D, C):
    """Contractions that end inside a 16-byte chunk and inside a 64-wide K
    block, with NaN in every padding element of dY's rows: the padding is
    read with the last chunk and must contribute nothing."""
    banner(f"dequantized backward, NaN row padding, N={N} D={D} C={C}")
    rng = np.random.default_rng(N * 11 + D + C)
    X = oracle.bf16_rne(rng.standard_normal((N, C)).astype(np.float32))
    W = oracle.bf16_rne((rng.standard_normal((D, C)) * 0.02).astype(np.float32))
    dY = oracle.bf16_rne((rng.standard_normal((N, D)) * 1e-3).astype(np.float32))
    ld = (D + 7) // 8 * 8 + 8
    buf = torch.full((N, ld), float("nan"), dtype=torch.bfloat16, device="cuda")
    buf[:, :D] = dev(dY)
    dYd = buf[:, :D]
    xq, xs = oracle.quant_1x128(X)
    wq, ws, _ = oracle.quant_128x128(W, with_transpose=False)
    dx = host(fb.fp8_dequant_gemm_dgrad(dYd, dev(wq), dev(ws), fb.FP8B_SCALE_BLOCKS_128X128, N, D, C))
    assert np.all(np.isfinite(dx))
    e = oracle.rel_row_error(dx, oracle.bf16_matmul(dY, oracle.dequant_bf16_128x128(wq, ws, D, C)))
    banner(f"  dgrad {e:.3e}")
    assert e <= TOL
    dw = host(fb.fp8_dequant_gemm_wgrad(dYd, dev(xq), dev(xs), fb.FP8B_SCALE_ROWS_1X128, N, D, C,
                                        out_dtype=torch.float32))
    assert np.all(np.isfinite(dw))
    e = oracle.rel_row_error(dw, oracle.bf16_matmul(np.ascontiguousarray(dY.T), oracle.dequant_bf16_rows(xq, xs, C)))
    banner(f"  wgrad {e:.3e}")
    assert e <= 1e-5


def test_dequant_backward_training_shape_every_tile():
    """The training layer's backward in the dequantized mode, at full size:
    DGrad on the forward's 128x128 W codes, WGrad on the forward's 1x128 X
    codes (from the GPU quantizers, as a layer runs them), checked on one
    row of every 256-row output tile (every output tile has a checked row)."""
    w = wl.train(0)
    N, C, D = w["N"], w["C"], w["D"]
    banner("dequantized backward at the training shape")
    xq, xs = fb.fp8_quantize_act_1x128(dev(w["X"]))
    wq, ws, _ = fb.fp8_quantize_weight_128x128(dev(w["W"]), transpose=False)
    dYd = dev(w["dY"])
    dx = host(fb.fp8_dequant_gemm_dgrad(dYd, wq, ws, fb.FP8B_SCALE_BLOCKS_128X128, N, D, C))
    dw = host(fb.fp8_dequant_gemm_wgrad(dYd, xq, xs, fb.FP8B_SCALE_ROWS_1X128, N, D, C))
    rows = tile_rows(N, 72)
    drows = tile_rows(D, 74)
    owq, ows, _ = oracle.quant_128x128(w["W"], with_transpose=False)
    e = oracle.rel_row_error(dx[rows], oracle.bf16_matmul(w["dY"][rows], oracle.dequant_bf16_128x128(owq, ows, D, C)))
    banner(f"  dgrad sampled rows {e:.3e}")
    assert e <= TOL
    oxq, oxs = oracle.quant_1x128(w["X"])
    xdeq = oracle.dequant_bf16_rows(oxq, oxs, C)
    e = oracle.rel_row_error(dw[drows], oracle.bf16_matmul(np.ascontiguousarray(w["dY"][:, drows].T), xdeq))
    banner(f"  wgrad sampled rows {e:.3e}")
    assert e <= TOL


def test_dequantized_backward_error_against_fp8_backward():
    """What the mode buys: DGrad and WGrad error against the exact binary64
    product of the bf16 inputs (512 training rows, sampled output rows), for
    the FP8 backward (dY quantized, FP8 GEMMs) and the dequantized backward
    (dY in bf16, forward codes dequantized).  The dequantized backward keeps
    dY exact, so its error must not exceed the FP8 backward's."""
    w = wl.train(0, rows=512)
    X, W, dY = w["X"], w["W"], w["dY"]
    N, C = X.shape
    D = W.shape[0]
    banner("backward error: FP8 GEMMs against bf16 GEMMs on dequantized operands")
    xd, wd, gd = dev(X), dev(W), dev(dY)
    xqT, xsT, xq, xs = fb.fp8_quantize_transposed(xd, rowwise=True)
    gqT, gsT, gq, gs = fb.fp8_quantize_transposed(gd, rowwise=True)
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(wd)
    f32 = torch.float32
    dx8 = host(fb.fp8_gemm_dgrad(gq, gs, wqT, ws, N, D, C, out_dtype=f32))
    dw8 = host(fb.fp8_gemm_wgrad(gqT, gsT, xqT, xsT, N, D, C, out_dtype=f32))
    dxb = host(fb.fp8_dequant_gemm_dgrad(gd, wq, ws, fb.FP8B_SCALE_BLOCKS_128X128, N, D, C))
    dwb = host(fb.fp8_dequant_gemm_wgrad(gd, xq, xs, fb.FP8B_SCALE_ROWS_1X128, N, D, C, out_dtype=f32))
    rng = np.random.default_rng(73)
    rows = np.sort(rng.choice(N, 64, replace=False))
    drows = np.sort(rng.choice(D, 64, replace=False))
    f64 = lambda b: wl.bf16_bits_to_f32(b).astype(np.float64)
    exact_dx = f64(dY[rows]) @ f64(W)
    exact_dw = f64(dY[:, drows]).T @ f64(X)
    e = {"dgrad_fp8": oracle.rel_row_error(dx8[rows], exact_dx),
         "dgrad_deq": oracle.rel_row_error(dxb[rows], exact_dx),
         "wgrad_fp8": oracle.rel_row_error(dw8[drows], exact_dw),
         "wgrad_deq": oracle.rel_row_error(dwb[drows], exact_dw)}
    banner("max row error vs exact: " + ", ".join(f"{k} {v:.3e}" for k, v in e.items()))
    assert e["dgrad_deq"] <= e["dgrad_fp8"] and e["wgrad_deq"] <= e["wgrad_fp8"], e


def test_dequant_backward_empty_contraction_writes_zeros():
    """An empty contraction (D = 0 for DGrad, N = 0 for WGrad) writes zeros
    (with a fill kernel, not a memset) and leaves dW as it is with beta = 1."""
    N, D, C = 130, 200, 300
    banner("dequantized backward with an empty contraction")
    dx = fb._new_out(N, C, torch.bfloat16, torch.device("cuda")).fill_(7.0)
    fb.fp8_dequant_gemm_dgrad(torch.empty((N, 0), dtype=torch.bfloat16, device="cuda"),
                              torch.empty((0, 384), dtype=torch.uint8, device="cuda"),
                              torch.empty((0, 3), dtype=torch.float32, device="cuda"),
                              fb.FP8B_SCALE_BLOCKS_128X128, N, 0, C, dx=dx)
    assert torch.all(dx == 0)
    dy0 = torch.empty((0, D), dtype=torch.bfloat16, device="cuda")
    xq0 = torch.empty((0, 384), dtype=torch.uint8, device="cuda")
    xs0 = torch.empty((0, 3), dtype=torch.float32, device="cuda")
    dw = fb._new_out(D, C, torch.bfloat16, torch.device("cuda")).fill_(7.0)
    fb.fp8_dequant_gemm_wgrad(dy0, xq0, xs0, fb.FP8B_SCALE_ROWS_1X128, 0, D, C, dw=dw)
    assert torch.all(dw == 0)
    dw32 = fb._new_out(D, C, torch.float32, torch.device("cuda")).fill_(7.0)
    fb.fp8_dequant_gemm_wgrad(dy0, xq0, xs0, fb.FP8B_SCALE_ROWS_1X128, 0, D, C, dw=dw32, beta=1)
    assert torch.all(dw32 == 7.0)
