"""GPU parity of the block-scaled GEMMs (FProp, DGrad, WGrad, grouped MoE)
against the oracle.  Both sides start from the same seeded inputs; each
side quantizes with its own code and computes its own GEMMs.  Bar:
max |y - y_oracle| / ||y_oracle row||_2 <= 2e-3 (the bf16 output rounding
alone can reach 2^-9 of the row norm); fp32 outputs must in addition sit
within 2^-12 * sum_k |a_k b_k| of the oracle (the accumulation error scale
of the fp8 MFMA dot product), a bound that stays meaningful for short or
cancelling rows.

Full-size launches use exactly the kernels and tile configurations the
benchmark times, and the oracle covers every output: the training layer
(8192 x 4096 x 12288, three GEMMs), the decode FProp, and all 128 experts
of the MoE layer.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_02_amd as fb
import oracle
from block_scaled_fp8_02_amd import workloads as wl
from gpu_util import TOL, banner, dev, dev_strided, host

pytestmark = pytest.mark.gpu


def gpu_layer(X, W, dY, out_dtype=torch.bfloat16):
    N, C = X.shape
    D = W.shape[0]
    xd, wd, gd = dev_strided(X), dev_strided(W), dev_strided(dY)
    xq, xs = fb.fp8_quantize_act_1x128(xd)
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(wd)
    gq, gs = fb.fp8_quantize_act_1x128(gd)
    gqT, gsT, _, _ = fb.fp8_quantize_transposed(gd)
    xqT, xsT, _, _ = fb.fp8_quantize_transposed(xd)
    y = fb.fp8_gemm_fprop(xq, xs, wq, ws, N, D, C, out_dtype=out_dtype)
    dx = fb.fp8_gemm_dgrad(gq, gs, wqT, ws, N, D, C, out_dtype=out_dtype)
    dw = fb.fp8_gemm_wgrad(gqT, gsT, xqT, xsT, N, D, C, out_dtype=out_dtype)
    return host(y), host(dx), host(dw)


def oracle_layer(X, W, dY):
    N, C = X.shape
    D = W.shape[0]
    xq, xs = oracle.quant_1x128(X)
    wq, ws, _ = oracle.quant_128x128(W, with_transpose=False)
    gq, gs = oracle.quant_1x128(dY)
    gqT, gsT = oracle.quant_colwise(dY)
    xqT, xsT = oracle.quant_colwise(X)
    y = oracle.fprop(xq, xs, wq, ws, C)
    dx = oracle.dgrad(gq, gs, wq, ws, D, C)
    dw = oracle.wgrad(gqT, gsT, xqT, xsT, gqT.shape[1])
    return y, dx, dw


def check(got, want, tol, what):
    err = oracle.rel_row_error(got, want)
    banner(f"{what}: rel row error {err:.3e} (tol {tol:.0e})")
    assert err <= tol, f"{what}: {err}"


# Accumulation bound for fp32 outputs: |error| <= 2^-12 * sum_k |a_k b_k|.
# The fp8 MFMA forms each 128-wide block's dot product with a narrower
# internal sum than fp32 (measured: up to ~1e-4 of sum |a_k b_k| on one
# block); promoting every block's partial sum into an fp32 accumulator with
# its scales, as the pages' GEMMs do, keeps the error at that level instead
# of letting it grow with K.
ACC_BOUND = 2.0 ** -12


def abs_products(X, W, dY):
    """sum_k |a_k b_k| for every output of the three GEMMs (fp64, oracle
    dequantization): the scale of the rounding error of any fp32 sum."""
    N, C = X.shape
    D = W.shape[0]
    xq, xs = oracle.quant_1x128(X)
    wq, ws, _ = oracle.quant_128x128(W, with_transpose=False)
    gq, gs = oracle.quant_1x128(dY)
    gqT, gsT = oracle.quant_colwise(dY)
    xqT, xsT = oracle.quant_colwise(X)
    K = gqT.shape[1]
    Xa = np.abs(oracle.deq_rowgroups(xq, xs, C))
    Wa = np.abs(oracle.deq_128x128(wq, ws, D, C))
    Ga = np.abs(oracle.deq_rowgroups(gq, gs, D))
    GTa = np.abs(oracle.deq_rowgroups(gqT, gsT, K))
    XTa = np.abs(oracle.deq_rowgroups(xqT, xsT, K))
    return (oracle.matmul_f64(Xa, Wa.T), oracle.matmul_f64(Ga, Wa), oracle.matmul_f64(GTa, XTa.T))


def check_f32(got, want, mag, what):
    """fp32 output: the row-norm error metric, and every element within
    the fp32 accumulation bound of the oracle."""
    err = oracle.rel_row_error(got, want)
    ratio = float(np.max(np.abs(got - want) / np.maximum(mag, 1e-300)))
    banner(f"{what}: rel row error {err:.3e}, |err|/sum|ab| {ratio:.3e} (bound {ACC_BOUND:.1e})")
    assert err <= TOL, f"{what}: {err}"
    assert ratio <= ACC_BOUND, f"{what}: {ratio}"


def test_tiny_workload_layer():
    w = wl.tiny(0)
    banner("tiny layer: FProp/DGrad/WGrad")
    ref = oracle_layer(w["X"], w["W"], w["dY"])
    got = gpu_layer(w["X"], w["W"], w["dY"], out_dtype=torch.bfloat16)
    for g, r, name in zip(got, ref, ("fprop", "dgrad", "wgrad")):
        check(g, r, TOL, f"tiny {name} bf16")
    mags = abs_products(w["X"], w["W"], w["dY"])
    got = gpu_layer(w["X"], w["W"], w["dY"], out_dtype=torch.float32)
    for g, r, m, name in zip(got, ref, mags, ("fprop", "dgrad", "wgrad")):
        check_f32(g, r, m, f"tiny {name} f32")


@pytest.mark.parametrize("N,D,C", [(1, 16, 1), (3, 130, 300), (200, 300, 260), (320, 400, 640),
                                   (129, 1, 129), (64, 256, 8), (257, 384, 1024)])
def test_ragged_layers(N, D, C):
    banner(f"ragged layer N={N} D={D} C={C}")
    rng = np.random.default_rng(N * 7 + D * 3 + C)
    X = (rng.standard_normal((N, C)) * np.exp(rng.uniform(-3, 3, (N, 1)))).astype(np.float32)
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    dY = (rng.standard_normal((N, D)) * 1e-3).astype(np.float32)
    ref = oracle_layer(X, W, dY)
    mags = abs_products(X, W, dY)
    got = gpu_layer(X, W, dY, out_dtype=torch.float32)
    for g, r, m, name in zip(got, ref, mags, ("fprop", "dgrad", "wgrad")):
        check_f32(g, r, m, f"ragged {name}")


SPLIT_SHAPES = [(64, 4096, 512), (37, 2304, 300), (1, 3000, 4100), (64, 24576, 384),
                # C % 4 != 0 (the ordered sum's partial-quad tail) and ragged D
                (37, 2304, 301), (1, 3000, 4099), (5, 2050, 130), (64, 24576, 4096)]


@pytest.mark.parametrize("N,D,C", SPLIT_SHAPES)
def test_dgrad_k_split(N, D, C):
    """Few token rows with a long contraction: DGrad runs as K ranges of
    fp32 partial sums plus an ordered sum of the ranges.  fp32 and bf16
    outputs against the oracle (the same bounds as every GEMM), the plain
    single-range entry point against the oracle too, and the split form
    repeated bit for bit.  The split partition is a function of the shape
    alone, so it applies to these shapes on any device."""
    banner(f"dgrad K split N={N} D={D} C={C}")
    assert fb.lib().fp8_gemm_dgrad_split_bytes(N, D, C) > 0
    rng = np.random.default_rng(N * 5 + D + C * 11)
    X = rng.standard_normal((N, C)).astype(np.float32)
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    dY = (rng.standard_normal((N, D)) * np.exp(rng.uniform(-4, 2, (1, D)))).astype(np.float32)
    ogq, ogs = oracle.quant_1x128(dY)
    owq, ows, _ = oracle.quant_128x128(W, with_transpose=False)
    want = oracle.dgrad(ogq, ogs, owq, ows, D, C)
    mag = abs_products(X, W, dY)[1]
    gq, gs = fb.fp8_quantize_act_1x128(dev_strided(dY))
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(dev_strided(W))
    f32 = torch.float32
    dx = fb.fp8_gemm_dgrad(gq, gs, wqT, ws, N, D, C, out_dtype=f32)
    check_f32(host(dx), want, mag, "split dgrad f32")
    again = fb.fp8_gemm_dgrad(gq, gs, wqT, ws, N, D, C, out_dtype=f32)
    assert torch.equal(dx, again), "split dgrad is not repeatable"
    # the caller's workspace (nothing allocated in the call), a short one refused
    work = fb.dgrad_split_workspace(N, D, C, gq.device)
    assert torch.equal(fb.fp8_gemm_dgrad(gq, gs, wqT, ws, N, D, C, out_dtype=f32, work=work), dx)
    with pytest.raises(ValueError):
        fb.fp8_gemm_dgrad(gq, gs, wqT, ws, N, D, C, out_dtype=f32, work=work[:-16])
    check(host(fb.fp8_gemm_dgrad(gq, gs, wqT, ws, N, D, C)), want, TOL, "split dgrad bf16")
    plain = fb._new_out(N, C, f32, gq.device)
    fb._call("fp8_gemm_dgrad", fb._ptr(gq), fb._ld(gq), fb._ptr(gs), fb._ld(gs), fb._ptr(wqT), fb._ld(wqT),
             fb._ptr(ws), fb._ld(ws), fb._ptr(plain), 0, fb._ld(plain), N, D, C, fb._stream(gq.device))
    check_f32(host(plain), want, mag, "single-range dgrad f32")


@pytest.mark.parametrize("N,D,C", SPLIT_SHAPES)
def test_mx_dgrad_k_split(N, D, C):
    """The MX DGrad on the same few-row shapes, split along K: against the
    MX oracle with the row-norm bar and the fp32 accumulation bound, and
    repeated bit for bit."""
    banner(f"mx dgrad K split N={N} D={D} C={C}")
    rng = np.random.default_rng(N * 3 + D * 7 + C)
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    dY = (rng.standard_normal((N, D)) * np.exp(rng.uniform(-4, 2, (1, D)))).astype(np.float32)
    ogq, oge = oracle.mx_quant_rows(dY)
    owqT, oweT = oracle.mx_quant_cols(W)
    want = oracle.mx_gemm(ogq, oge, owqT, oweT, D)
    mag = oracle.matmul_f64(np.abs(oracle.deq_mx(ogq, oge, D)), np.abs(oracle.deq_mx(owqT, oweT, D)).T)
    gq, ge, _, _ = fb.fp8_mx_quantize_1x32(dev_strided(dY), rowwise=True, colwise=False)
    _, _, wqT, weT = fb.fp8_mx_quantize_1x32(dev_strided(W), rowwise=False, colwise=True)
    dx = fb.fp8_mx_gemm_dgrad(gq, ge, wqT, weT, N, D, C, out_dtype=torch.float32)
    check_f32(host(dx), want, mag, "mx split dgrad f32")
    again = fb.fp8_mx_gemm_dgrad(gq, ge, wqT, weT, N, D, C, out_dtype=torch.float32)
    assert torch.equal(dx, again), "mx split dgrad is not repeatable"
    work = fb.dgrad_split_workspace(N, D, C, gq.device)
    assert torch.equal(fb.fp8_mx_gemm_dgrad(gq, ge, wqT, weT, N, D, C, out_dtype=torch.float32, work=work), dx)
    check(host(fb.fp8_mx_gemm_dgrad(gq, ge, wqT, weT, N, D, C)), want, TOL, "mx split dgrad bf16")


@pytest.mark.parametrize("N,D,C", [(65, 4096, 512), (64, 1920, 512)])
def test_dgrad_split_entry_without_split_is_plain_dgrad(N, D, C):
    """Where no split applies (more than 64 rows; fewer than 16 K blocks)
    the split entry points run the plain DGrad: bit for bit the same output,
    with no workspace at all."""
    banner(f"dgrad split entry, no split: N={N} D={D} C={C}")
    assert fb.lib().fp8_gemm_dgrad_split_bytes(N, D, C) == 0
    rng = np.random.default_rng(N + D + C)
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    dY = (rng.standard_normal((N, D)) * 1e-3).astype(np.float32)
    gq, gs = fb.fp8_quantize_act_1x128(dev_strided(dY))
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(dev_strided(W))
    gmq, gme, _, _ = fb.fp8_mx_quantize_1x32(dev(dY), rowwise=True, colwise=False)
    _, _, wmqT, wmeT = fb.fp8_mx_quantize_1x32(dev(W), rowwise=False, colwise=True)
    for plain_fn, split_fn, a, sa, b, sb in (("fp8_gemm_dgrad", "fp8_gemm_dgrad_split", gq, gs, wqT, ws),
                                             ("fp8_mx_gemm_dgrad", "fp8_mx_gemm_dgrad_split", gmq, gme, wmqT, wmeT)):
        outs = []
        for fn, extra in ((plain_fn, ()), (split_fn, (None, 0))):
            dx = fb._new_out(N, C, torch.float32, a.device).fill_(float("nan"))
            fb._call(fn, fb._ptr(a), fb._ld(a), fb._ptr(sa), fb._ld(sa), fb._ptr(b), fb._ld(b),
                     fb._ptr(sb), fb._ld(sb), fb._ptr(dx), 0, fb._ld(dx), N, D, C, *extra, fb._stream(a.device))
            outs.append(dx)
        assert torch.equal(outs[0], outs[1]), f"{split_fn} without a split differs from {plain_fn}"


def test_zero_contraction_gives_zero():
    """C = 0: every output is an empty sum."""
    xq = torch.zeros((5, 16), dtype=torch.uint8, device="cuda")[:, :0]
    xs = torch.zeros((5, 4), dtype=torch.float32, device="cuda")[:, :0]
    wq = torch.zeros((7, 16), dtype=torch.uint8, device="cuda")[:, :0]
    ws = torch.zeros((1, 4), dtype=torch.float32, device="cuda")[:, :0]
    y = torch.full((5, 8), 3.0, dtype=torch.float32, device="cuda")[:, :7]
    fb.fp8_gemm_fprop(xq, xs, wq, ws, 5, 7, 0, y=y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def test_decode_fprop_full():
    w = wl.decode(0)
    banner("decode FProp 64x24576x4096 (full, oracle full)")
    X, W = w["X"], w["W"]
    xq, xs = fb.fp8_quantize_act_1x128(dev(X))
    wq, ws, _ = fb.fp8_quantize_weight_128x128(dev(W), transpose=False)
    y = host(fb.fp8_gemm_fprop(xq, xs, wq, ws, 64, 24576, 4096))
    wp, _ = fb.fp8_pack_decode_weight(wq, 24576, 4096)
    y_dec = host(fb.fp8_gemm_fprop_decode(xq, xs, wp, ws, 64, 24576, 4096))
    assert np.array_equal(y_dec.view(np.uint32), y.view(np.uint32))     # the packed weight, bit for bit
    oxq, oxs = oracle.quant_1x128(X)
    owq, ows, _ = oracle.quant_128x128(W, with_transpose=False)
    check(y, oracle.fprop(oxq, oxs, owq, ows, 4096), TOL, "decode fprop")


@pytest.fixture(scope="module")
def train_full():
    """The three training GEMMs at full size (8192 x 4096 x 12288) from the
    GPU's own quantizers, in the launch configuration the benchmark times;
    outputs kept on the host for the full-size oracle comparisons below."""
    w = wl.train(0)
    X, W, dY = w["X"], w["W"], w["dY"]
    N, C, D = 8192, 12288, 4096
    banner("train: GPU quantize + FProp/DGrad/WGrad at full size")
    xd, wd, gd = dev(X), dev(W), dev(dY)
    xqT, xsT, xq, xs = fb.fp8_quantize_transposed(xd, rowwise=True)
    gqT, gsT, gq, gs = fb.fp8_quantize_transposed(gd, rowwise=True)
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(wd)
    y = host(fb.fp8_gemm_fprop(xq, xs, wq, ws, N, D, C))
    dx = host(fb.fp8_gemm_dgrad(gq, gs, wqT, ws, N, D, C))
    dw = host(fb.fp8_gemm_wgrad(gqT, gsT, xqT, xsT, N, D, C))
    del xd, wd, gd, xqT, xsT, xq, xs, gqT, gsT, gq, gs, wq, ws, wqT
    torch.cuda.empty_cache()
    return {"w": w, "y": y, "dx": dx, "dw": dw}


def test_train_fprop_full(train_full):
    """Training FProp, every output against the oracle (full size)."""
    w = train_full["w"]
    banner("train fprop: oracle on the full output")
    oxq, oxs = oracle.quant_1x128(w["X"])
    owq, ows, _ = oracle.quant_128x128(w["W"], with_transpose=False)
    check(train_full["y"], oracle.fprop(oxq, oxs, owq, ows, 12288), TOL, "train fprop (full)")


def test_train_dgrad_full(train_full):
    """Training DGrad, every output against the oracle (full size)."""
    w = train_full["w"]
    banner("train dgrad: oracle on the full output")
    ogq, ogs = oracle.quant_1x128(w["dY"])
    owq, ows, _ = oracle.quant_128x128(w["W"], with_transpose=False)
    check(train_full["dx"], oracle.dgrad(ogq, ogs, owq, ows, 4096, 12288), TOL, "train dgrad (full)")


def test_train_wgrad_full(train_full):
    """Training WGrad, every output against the oracle (full size)."""
    w = train_full["w"]
    banner("train wgrad: oracle on the full output")
    ogqT, ogsT = oracle.quant_colwise(w["dY"])
    oxqT, oxsT = oracle.quant_colwise(w["X"])
    check(train_full["dw"], oracle.wgrad(ogqT, ogsT, oxqT, oxsT, 8192), TOL, "train wgrad (full)")


def test_unified_forward_is_batch_invariant():
    """Rollout FProp of 64 tokens equals rows 0..63 of the training-size
    FProp bit for bit, with the decode weight (Jet-RL notes, section 4.1:
    rollout runs the training forward's own FP8 computation)."""
    w = wl.decode(0)
    rng = wl.rng_for(7)
    X = wl.normal(rng, (8192, 4096), 1.0)
    wl.add_outlier_channels(rng, X)
    X = wl.f32_to_bf16_bits(X)
    banner("batch invariance 64 vs 8192 rows")
    wq, ws, _ = fb.fp8_quantize_weight_128x128(dev(w["W"]), transpose=False)
    xq, xs = fb.fp8_quantize_act_1x128(dev(X))
    # the full weight and a ragged one (its last tile 88 rows): the decode
    # tiles (64 x 128, 64 x 32, 64 x 16) against the 256 x 256 training tile
    for D in (24576, 24536, 16384, 4000):
        y_big = fb.fp8_gemm_fprop(xq, xs, wq[:D], ws, 8192, D, 4096)
        for m in (1, 17, 64, 100, 256):
            xqm, xsm = fb.fp8_quantize_act_1x128(dev(X[:m]))
            ym = fb.fp8_gemm_fprop(xqm, xsm, wq[:D], ws, m, D, 4096)
            assert torch.equal(ym, y_big[:m]), (D, m)
    y_again = fb.fp8_gemm_fprop(xq, xs, wq[:D], ws, 8192, D, 4096)
    assert torch.equal(y_again, y_big)


# Decode-shaped FProp (at most 64 token rows, a weight of at least 128 groups
# of 96 rows) runs on the weight-streaming decode kernel; these shapes give it
# a ragged last row group, contractions shorter than one staged chunk, a
# partial chunk and a partial register-ring group.
ROWS96_SHAPES = [(1, 12289, 1), (37, 12289, 300), (64, 12300, 1100), (17, 24576, 640),
                 (64, 12193, 4099)]


@pytest.mark.parametrize("M,D,C", ROWS96_SHAPES)
def test_decode_rows_kernel_ragged(M, D, C):
    banner(f"decode rows kernel M={M} D={D} C={C}")
    rng = np.random.default_rng(M * 5 + D + C)
    X = (rng.standard_normal((80, C)) * np.exp(rng.uniform(-3, 3, (80, 1)))).astype(np.float32)
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    wq, ws, _ = fb.fp8_quantize_weight_128x128(dev_strided(W), transpose=False)
    xq, xs = fb.fp8_quantize_act_1x128(dev_strided(X))
    y32 = host(fb.fp8_gemm_fprop(xq[:M], xs[:M], wq, ws, M, D, C, out_dtype=torch.float32))
    oxq, oxs = oracle.quant_1x128(X[:M])
    owq, ows, _ = oracle.quant_128x128(W, with_transpose=False)
    mag = oracle.matmul_f64(np.abs(oracle.deq_rowgroups(oxq, oxs, C)),
                            np.abs(oracle.deq_128x128(owq, ows, D, C)).T)
    check_f32(y32, oracle.fprop(oxq, oxs, owq, ows, C), mag, "decode rows fprop f32")
    # same rows as the 80-row call (training tiles), bit for bit, both outputs
    for dt in (torch.float32, torch.bfloat16):
        y_big = fb.fp8_gemm_fprop(xq, xs, wq, ws, 80, D, C, out_dtype=dt)
        y_m = fb.fp8_gemm_fprop(xq[:M], xs[:M], wq, ws, M, D, C, out_dtype=dt)
        assert torch.equal(y_m, y_big[:M]), dt


@pytest.mark.parametrize("N,D,C", [(37, 300, 12300), (64, 1100, 12193), (1, 128, 16500)])
def test_dgrad_on_decode_kernel(N, D, C):
    """Few-row DGrad with a wide output and a contraction too short to split
    runs on the weight-streaming decode kernel, which then reads the 128x128
    weight scales transposed (K block along the grid's rows): fp32 output
    against the oracle, both recipes."""
    banner(f"dgrad on the decode kernel N={N} D={D} C={C}")
    assert fb.lib().fp8_gemm_dgrad_split_bytes(N, D, C) == 0
    rng = np.random.default_rng(N + D + C)
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    dY = (rng.standard_normal((N, D)) * np.exp(rng.uniform(-2, 2, (N, 1)))).astype(np.float32)
    gq, gs = fb.fp8_quantize_act_1x128(dev_strided(dY))
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(dev_strided(W))
    dx = host(fb.fp8_gemm_dgrad(gq, gs, wqT, ws, N, D, C, out_dtype=torch.float32))
    ogq, ogs = oracle.quant_1x128(dY)
    owq, ows, _ = oracle.quant_128x128(W, with_transpose=False)
    mag = oracle.matmul_f64(np.abs(oracle.deq_rowgroups(ogq, ogs, D)), np.abs(oracle.deq_128x128(owq, ows, D, C)))
    check_f32(dx, oracle.dgrad(ogq, ogs, owq, ows, D, C), mag, "dgrad decode kernel f32")
    # MX: the row-wise E8M0 of W^T
    mgq, mge, _, _ = fb.fp8_mx_quantize_1x32(dev_strided(dY), colwise=False)
    _, _, mwqT, mweT = fb.fp8_mx_quantize_1x32(dev_strided(W), rowwise=False)
    mdx = host(fb.fp8_mx_gemm_dgrad(mgq, mge, mwqT, mweT, N, D, C, out_dtype=torch.float32))
    oq, oe = oracle.mx_quant_rows(dY)
    owqT, oweT = oracle.mx_quant_cols(W)
    ref = oracle.mx_gemm(oq, oe, owqT, oweT, D)
    mmag = oracle.matmul_f64(np.abs(oracle.deq_mx(oq, oe, D)), np.abs(oracle.deq_mx(owqT, oweT, D)).T)
    err = oracle.rel_row_error(mdx, ref)
    ratio = float(np.max(np.abs(mdx - ref) / np.maximum(mmag, 1e-300)))
    banner(f"mx dgrad decode kernel: {err:.3e}, |err|/sum|ab| {ratio:.3e}")
    assert err <= TOL and ratio <= ACC_BOUND


def packed_codes_ref(wq_host, D, C):
    """Decode layout of row-major codes, written out with numpy: per group
    of 16 rows and K block, half h holds chunks q + 4h of rows r at lane
    16q + r (rows past D zero)."""
    KB, R = (C + 127) // 128, (D + 15) // 16 * 16
    rows = np.zeros((R, KB * 128), np.uint8)
    rows[:D] = wq_host[:D, :KB * 128]
    t = rows.reshape(R // 16, 16, KB, 2, 4, 16)          # grp, r, k, h, q, byte
    return np.ascontiguousarray(t.transpose(0, 2, 3, 4, 1, 5)).reshape(R, KB * 128)


@pytest.mark.parametrize("D,C", [(1, 1), (17, 300), (100, 128), (37, 1100)])
def test_pack_decode_layout(D, C):
    rng = np.random.default_rng(D + C)
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    wq, ws, _ = fb.fp8_quantize_weight_128x128(dev_strided(W), transpose=False)
    wp, wep = fb.fp8_pack_decode_weight(wq, D, C)
    assert wep is None
    np.testing.assert_array_equal(host(wp), packed_codes_ref(host(wq), D, C))


# Decode FProp on the packed weight: bit for bit the row-major FProp (itself
# checked against the oracle above), at ragged shapes, few-row weights and
# the full decode weight, for both output types.
DECODE_SHAPES = [(1, 1, 1), (5, 17, 130), (64, 100, 4096), (37, 12289, 300), (64, 12300, 1100),
                 (17, 24576, 640), (64, 12193, 4099), (3, 2000, 8192)]


@pytest.mark.parametrize("M,D,C", DECODE_SHAPES)
def test_decode_packed_matches_fprop(M, D, C):
    banner(f"decode packed M={M} D={D} C={C}")
    rng = np.random.default_rng(M + 3 * D + C)
    X = (rng.standard_normal((M, C)) * np.exp(rng.uniform(-3, 3, (M, 1)))).astype(np.float32)
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    wq, ws, _ = fb.fp8_quantize_weight_128x128(dev_strided(W), transpose=False)
    xq, xs = fb.fp8_quantize_act_1x128(dev_strided(X))
    wp, _ = fb.fp8_pack_decode_weight(wq, D, C)
    for dt in (torch.float32, torch.bfloat16):
        y_row = fb.fp8_gemm_fprop(xq, xs, wq, ws, M, D, C, out_dtype=dt)
        y_dec = fb.fp8_gemm_fprop_decode(xq, xs, wp, ws, M, D, C, out_dtype=dt)
        assert torch.equal(y_dec, y_row), dt


def test_decode_packed_oracle_and_edges():
    """The packed decode against the oracle directly (fp32 output), more than
    64 tokens refused, an empty contraction written as zeros."""
    M, D, C = 64, 2000, 1100
    rng = np.random.default_rng(77)
    X = (rng.standard_normal((M, C)) * np.exp(rng.uniform(-3, 3, (M, 1)))).astype(np.float32)
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    wq, ws, _ = fb.fp8_quantize_weight_128x128(dev_strided(W), transpose=False)
    xq, xs = fb.fp8_quantize_act_1x128(dev_strided(X))
    wp, _ = fb.fp8_pack_decode_weight(wq, D, C)
    y = host(fb.fp8_gemm_fprop_decode(xq, xs, wp, ws, M, D, C, out_dtype=torch.float32))
    oxq, oxs = oracle.quant_1x128(X)
    owq, ows, _ = oracle.quant_128x128(W, with_transpose=False)
    mag = oracle.matmul_f64(np.abs(oracle.deq_rowgroups(oxq, oxs, C)), np.abs(oracle.deq_128x128(owq, ows, D, C)).T)
    check_f32(y, oracle.fprop(oxq, oxs, owq, ows, C), mag, "decode packed f32")
    X65 = dev(np.ones((65, C), np.float32))
    xq65, xs65 = fb.fp8_quantize_act_1x128(X65)
    with pytest.raises(RuntimeError):
        fb.fp8_gemm_fprop_decode(xq65, xs65, wp, ws, 65, D, C)
    z = torch.full((5, 8), 3.0, dtype=torch.float32, device="cuda")[:, :7]
    empty = torch.zeros((7, 16), dtype=torch.uint8, device="cuda")
    fb.fp8_gemm_fprop_decode(empty[:5, :0], torch.zeros((5, 4), dtype=torch.float32, device="cuda")[:, :0],
                             torch.zeros((16, 0), dtype=torch.uint8, device="cuda"),
                             torch.zeros((1, 4), dtype=torch.float32, device="cuda")[:, :0], 5, 7, 0, y=z)
    torch.cuda.synchronize()
    assert torch.all(z == 0)


def test_wgrad_accumulate_fp32():
    rng = np.random.default_rng(5)
    N, D, C = 384, 256, 512
    X = rng.standard_normal((N, C)).astype(np.float32)
    dY = (rng.standard_normal((N, D)) * 1e-3).astype(np.float32)
    gqT, gsT, _, _ = fb.fp8_quantize_transposed(dev(dY))
    xqT, xsT, _, _ = fb.fp8_quantize_transposed(dev(X))
    base = torch.from_numpy(rng.standard_normal((D, C)).astype(np.float32)).cuda()
    acc = base.clone()
    fb.fp8_gemm_wgrad(gqT, gsT, xqT, xsT, N, D, C, dw=acc, beta=1)
    plain = fb.fp8_gemm_wgrad(gqT, gsT, xqT, xsT, N, D, C, out_dtype=torch.float32)
    assert torch.equal(acc, base + plain)


# ----------------------------------------------------------------- MoE
def moe_gpu(w):
    """Grouped FProp/DGrad/WGrad for gate/up and down on the GPU."""
    offs = w["offsets"]
    E, I2, H = w["W_gu"].shape
    I = w["inter"]
    R = int(offs[-1])
    offs_d = dev(offs.astype(np.int32))
    out = {}
    Wgu = dev(w["W_gu"].reshape(E * I2, H))
    Wd = dev(w["W_d"].reshape(E * H, I))
    gu_q, gu_s, gu_qT = fb.fp8_quantize_weight_128x128(Wgu)
    d_q, d_s, d_qT = fb.fp8_quantize_weight_128x128(Wd)
    Xd, Ad, dHd, dYd = dev(w["X_perm"]), dev(w["A"]), dev(w["dH"]), dev(w["dY_d"])
    xqT, xsT, xq, xs = fb.fp8_quantize_transposed_grouped(Xd, offs_d, rowwise=True)
    aqT, asT, aq, as_ = fb.fp8_quantize_transposed_grouped(Ad, offs_d, rowwise=True)
    hqT, hsT, hq, hs = fb.fp8_quantize_transposed_grouped(dHd, offs_d, rowwise=True)
    yqT, ysT, yq, ys = fb.fp8_quantize_transposed_grouped(dYd, offs_d, rowwise=True)
    # gate/up: H -> 2I
    out["gu_fprop"] = fb.fp8_gemm_fprop_grouped(xq, xs, gu_q, I2 * gu_q.stride(0), gu_s,
                                                (I2 // 128) * gu_s.stride(0), offs_d, R, I2, H)
    out["gu_dgrad"] = fb.fp8_gemm_dgrad_grouped(hq, hs, gu_qT, I2, gu_s, (I2 // 128) * gu_s.stride(0),
                                                offs_d, R, I2, H)
    out["gu_wgrad"] = fb.fp8_gemm_wgrad_grouped(hqT, hsT, xqT, xsT, offs_d, R, I2, H)
    # down: I -> H
    out["d_fprop"] = fb.fp8_gemm_fprop_grouped(aq, as_, d_q, H * d_q.stride(0), d_s,
                                               (H // 128) * d_s.stride(0), offs_d, R, H, I)
    out["d_dgrad"] = fb.fp8_gemm_dgrad_grouped(yq, ys, d_qT, H, d_s, (H // 128) * d_s.stride(0),
                                               offs_d, R, H, I)
    out["d_wgrad"] = fb.fp8_gemm_wgrad_grouped(yqT, ysT, aqT, asT, offs_d, R, H, I)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


@pytest.fixture(scope="module")
def moe_full():
    w = wl.moe(0)
    banner("moe: grouped GEMMs at full size")
    return w, moe_gpu(w)


@pytest.mark.parametrize("proj", ["gu", "d"])
def test_moe_grouped_full_every_expert(moe_full, proj):
    """All six grouped GEMMs of the MoE layer at full size (4096 tokens,
    top-8 of 128 experts): every expert's rows and weight gradient against
    the oracle run on that expert alone."""
    w, got = moe_full
    offs = w["offsets"]
    I = w["inter"]
    banner(f"moe {proj}: oracle on all {w['experts']} experts")
    worst = {"fprop": 0.0, "dgrad": 0.0, "wgrad": 0.0}
    for e in range(w["experts"]):
        a, b = int(offs[e]), int(offs[e + 1])
        if proj == "gu":
            Xn, Wn, dYn = w["X_perm"][a:b], w["W_gu"][e], w["dH"][a:b]
        else:
            Xn, Wn, dYn = w["A"][a:b], w["W_d"][e], w["dY_d"][a:b]
        y, dx, dw = oracle_layer(Xn, Wn, dYn)
        for name, g, r in (("fprop", got[f"{proj}_fprop"][a:b], y), ("dgrad", got[f"{proj}_dgrad"][a:b], dx),
                           ("wgrad", got[f"{proj}_wgrad"][e], dw)):
            err = oracle.rel_row_error(g, r)
            assert err <= TOL, f"moe e{e} ({b - a} rows) {proj} {name}: {err}"
            worst[name] = max(worst[name], err)
    banner(f"moe {proj}: worst rel row error over the experts " +
           ", ".join(f"{k} {v:.3e}" for k, v in worst.items()))


def test_moe_grouped_edge_segments():
    banner("grouped GEMMs with empty and tiny experts")
    rng = np.random.default_rng(11)
    offs = np.array([0, 0, 1, 129, 129, 400, 700, 700], dtype=np.int32)
    E, R, H, Dn = 7, 700, 256, 128
    X = rng.standard_normal((R, H)).astype(np.float32)
    dY = (rng.standard_normal((R, Dn)) * 1e-3).astype(np.float32)
    Ws = (rng.standard_normal((E, Dn, H)) * 0.02).astype(np.float32)
    offs_d = dev(offs)
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(dev(Ws.reshape(E * Dn, H)))
    xqT, xsT, xq, xs = fb.fp8_quantize_transposed_grouped(dev(X), offs_d, rowwise=True)
    gqT, gsT, gq, gs = fb.fp8_quantize_transposed_grouped(dev(dY), offs_d, rowwise=True)
    y = host(fb.fp8_gemm_fprop_grouped(xq, xs, wq, Dn * wq.stride(0), ws, ws.stride(0), offs_d, R, Dn, H,
                                       out_dtype=torch.float32))
    dx = host(fb.fp8_gemm_dgrad_grouped(gq, gs, wqT, Dn, ws, ws.stride(0), offs_d, R, Dn, H,
                                        out_dtype=torch.float32))
    dw = host(fb.fp8_gemm_wgrad_grouped(gqT, gsT, xqT, xsT, offs_d, R, Dn, H, out_dtype=torch.float32))
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if b == a:
            assert np.all(dw[e] == 0)
            continue
        ry, rdx, rdw = oracle_layer(X[a:b], Ws[e], dY[a:b])
        my, mdx, mdw = abs_products(X[a:b], Ws[e], dY[a:b])
        check_f32(y[a:b], ry, my, f"edge e{e} fprop")
        check_f32(dx[a:b], rdx, mdx, f"edge e{e} dgrad")
        check_f32(dw[e], rdw, mdw, f"edge e{e} wgrad")


def test_moe_grouped_tail_boundaries():
    """Row-grouped FProp and DGrad run an expert's whole 256-row tiles in one
    launch and a remainder of at most 64 rows in a second one: experts ending
    0, 1, 63, 64 and 65 rows past a whole tile, experts of fewer than 64 rows,
    and empty ones, each against the oracle."""
    banner("grouped GEMMs: remainders around the 64-row split")
    rng = np.random.default_rng(12)
    counts = np.array([64, 65, 256, 257, 320, 321, 0, 63, 576, 577, 1, 128, 0, 319], dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    E, R, H, Dn = len(counts), int(offs[-1]), 384, 384
    X = rng.standard_normal((R, H)).astype(np.float32)
    dY = (rng.standard_normal((R, Dn)) * 1e-3).astype(np.float32)
    Ws = (rng.standard_normal((E, Dn, H)) * 0.02).astype(np.float32)
    offs_d = dev(offs)
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(dev(Ws.reshape(E * Dn, H)))
    _, _, xq, xs = fb.fp8_quantize_transposed_grouped(dev(X), offs_d, rowwise=True)
    _, _, gq, gs = fb.fp8_quantize_transposed_grouped(dev(dY), offs_d, rowwise=True)
    sw = (Dn // 128) * ws.stride(0)
    y32 = fb.fp8_gemm_fprop_grouped(xq, xs, wq, Dn * wq.stride(0), ws, sw, offs_d, R, Dn, H,
                                    out_dtype=torch.float32)
    dx32 = fb.fp8_gemm_dgrad_grouped(gq, gs, wqT, Dn, ws, sw, offs_d, R, Dn, H, out_dtype=torch.float32)
    ybf = fb.fp8_gemm_fprop_grouped(xq, xs, wq, Dn * wq.stride(0), ws, sw, offs_d, R, Dn, H)
    dxbf = fb.fp8_gemm_dgrad_grouped(gq, gs, wqT, Dn, ws, sw, offs_d, R, Dn, H)
    torch.cuda.synchronize()
    # the bf16 outputs (staged epilogue) are the fp32 outputs (direct stores) rounded
    assert torch.equal(ybf.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(dxbf.view(torch.int16), dx32.to(torch.bfloat16).view(torch.int16))
    y, dx = host(y32), host(dx32)
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if b == a:
            continue
        ry, rdx, _ = oracle_layer(X[a:b], Ws[e], dY[a:b])
        my, mdx, _ = abs_products(X[a:b], Ws[e], dY[a:b])
        check_f32(y[a:b], ry, my, f"tail e{e} ({b - a} rows) fprop")
        check_f32(dx[a:b], rdx, mdx, f"tail e{e} ({b - a} rows) dgrad")


def _wgrad_grouped_both_outputs(gqT, gsT, xqT, xsT, offs_d, R, Dn, C):
    """The grouped WGrad twice: bf16 output (staged through the LDS at each
    expert boundary) and fp32 output (stored from the registers)."""
    bf = fb.fp8_gemm_wgrad_grouped(gqT, gsT, xqT, xsT, offs_d, R, Dn, C)
    f32 = fb.fp8_gemm_wgrad_grouped(gqT, gsT, xqT, xsT, offs_d, R, Dn, C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return bf, f32


def test_moe_wgrad_bf16_matches_fp32_path(moe_full):
    """Both MoE weight gradients at full size: the bf16 result is the fp32
    result rounded to nearest-even, bit for bit (the arithmetic per output
    is the same; only the way the tile leaves differs)."""
    w, _ = moe_full
    offs = w["offsets"]
    E, I2, H = w["W_gu"].shape
    I = w["inter"]
    R = int(offs[-1])
    offs_d = dev(offs.astype(np.int32))
    for name, g, x, Dn, C in (("gu", w["dH"], w["X_perm"], I2, H), ("d", w["dY_d"], w["A"], H, I)):
        banner(f"moe {name} wgrad: bf16 output against fp32 output")
        gqT, gsT, _, _ = fb.fp8_quantize_transposed_grouped(dev(g), offs_d, rowwise=True)
        xqT, xsT, _, _ = fb.fp8_quantize_transposed_grouped(dev(x), offs_d, rowwise=True)
        bf, f32 = _wgrad_grouped_both_outputs(gqT, gsT, xqT, xsT, offs_d, R, Dn, C)
        assert torch.equal(bf.view(torch.int16), f32.to(torch.bfloat16).view(torch.int16)), name
        del bf, f32


@pytest.mark.parametrize("seed,E,Dn,C", [(3, 200, 1024, 1024), (4, 61, 256, 768), (5, 9, 512, 256)])
def test_moe_wgrad_many_experts_per_block(seed, E, Dn, C):
    """Full-tile grouped WGrads with several experts per block, empty
    experts, one-row experts and experts past a 128-row boundary: bf16
    output equal to the fp32 output rounded, bit for bit, and the fp32
    output within the accumulation bound of the oracle on sampled experts."""
    banner(f"grouped wgrad, many experts per block: seed {seed} E {E} {Dn}x{C}")
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, 300, size=E)
    counts[rng.choice(E, size=max(1, E // 6), replace=False)] = 0
    counts[rng.choice(E, size=max(1, E // 8), replace=False)] = 1
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offs[-1])
    X = rng.standard_normal((R, C)).astype(np.float32)
    dY = (rng.standard_normal((R, Dn)) * 1e-3).astype(np.float32)
    offs_d = dev(offs)
    xqT, xsT, _, _ = fb.fp8_quantize_transposed_grouped(dev(X), offs_d, rowwise=True)
    gqT, gsT, _, _ = fb.fp8_quantize_transposed_grouped(dev(dY), offs_d, rowwise=True)
    bf, f32 = _wgrad_grouped_both_outputs(gqT, gsT, xqT, xsT, offs_d, R, Dn, C)
    assert torch.equal(bf.view(torch.int16), f32.to(torch.bfloat16).view(torch.int16))
    dw = host(f32)
    for e in sorted(set(rng.choice(E, size=4, replace=False).tolist()) | {int(np.argmax(counts))}):
        a, b = int(offs[e]), int(offs[e + 1])
        if b == a:
            assert np.all(dw[e] == 0), f"empty expert {e}"
            continue
        gq, gs = oracle.quant_colwise(dY[a:b])
        xq, xs = oracle.quant_colwise(X[a:b])
        ref = oracle.wgrad(gq, gs, xq, xs, b - a)
        mag = oracle.matmul_f64(np.abs(oracle.deq_rowgroups(gq, gs, b - a)),
                                np.abs(oracle.deq_rowgroups(xq, xs, b - a)).T)
        check_f32(dw[e], ref, mag, f"grouped wgrad e{e} ({b - a} rows)")
