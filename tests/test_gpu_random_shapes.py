"""A seeded sweep of random small shapes through every quantizer and the
three GEMMs, and the fused producers, against the oracle: codes and scales bit for bit (1x128 rows,
128x128 weight blocks with the transposed codes, the token-axis dual
quantizer, MXFP8 in both orientations), GEMM fp32 outputs within the row-norm
tolerance and the fp8 accumulation bound.  The accumulation bound holds for
every output; the row-norm tolerance is checked where a row has at least 16
outputs: with fewer, the row norm can be a single sum that these inputs
cancel to a fraction of a percent of its sum |a_k b_k|, and a relative
error of that one sum measures the cancellation, not the GEMM (measured with
element-wise magnitudes over three decades: D = 1, C = 292, worst row 0.23%
of its sum |a_k b_k|, error 1.3e-5 of it).
Shapes mix sizes below, at and
just past the 32-, 128- and 256-element boundaries; activations and
gradients are Gaussian rows whose magnitudes spread over three decades, with
outlier channels, as in the workloads."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_02_amd as fb
import oracle
from gpu_util import TOL, assert_bytes_equal, assert_scales_equal, banner, dev_strided, host

pytestmark = pytest.mark.gpu

# Element bound for fp32 outputs: 2^-11 * sum_k |a_k b_k|.  The fp8 MFMA sums
# each 128-wide block with a narrower internal precision than fp32; with
# outlier channels (x50) sharing a block with ordinary values its error on one
# block was measured at up to 2.8e-4 of sum |a_k b_k| (DGrad, D = 33: a single
# partial block), above the 2^-12 that inputs without outliers stay within.
ACC_BOUND = 2.0 ** -11
EDGES = [1, 2, 31, 32, 33, 127, 128, 129, 255, 256, 257]


def _shapes(seed: int, n: int):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dims = [int(rng.choice(EDGES)) if rng.random() < 0.5 else int(rng.integers(1, 300)) for _ in range(3)]
        out.append(tuple(dims))
    return out


SHAPES = _shapes(2024, 16)


def _data(rng, shape, spread=3.0):
    """Gaussian rows with magnitudes spread over three decades, and 1% of
    the columns (at least one) scaled x50, as the workloads' outlier
    channels."""
    rows, cols = shape
    x = rng.standard_normal(shape) * np.exp(rng.uniform(-spread, spread, (rows, 1)))
    hot = rng.choice(cols, max(1, round(0.01 * cols)), replace=False)
    x[:, hot] *= 50.0
    return x.astype(np.float32)


@pytest.mark.parametrize("N,D,C", SHAPES)
def test_random_shape_quantizers_and_gemms(N, D, C):
    banner(f"random shape N={N} D={D} C={C}")
    rng = np.random.default_rng(N * 1000003 + D * 1009 + C)
    X = _data(rng, (N, C))
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    dY = (_data(rng, (N, D)) * 1e-3).astype(np.float32)
    xd, wd, gd = dev_strided(X), dev_strided(W), dev_strided(dY)

    # quantizers
    xqT, xsT, xq, xs = fb.fp8_quantize_transposed(xd, rowwise=True)
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(wd)
    gq, gs = fb.fp8_quantize_act_1x128(gd)
    gqT, gsT, _, _ = fb.fp8_quantize_transposed(gd)
    oxq, oxs = oracle.quant_1x128(X)
    oxqT, oxsT = oracle.quant_colwise(X)
    owq, ows, owqT = oracle.quant_128x128(W)
    ogq, ogs = oracle.quant_1x128(dY)
    ogqT, ogsT = oracle.quant_colwise(dY)
    for got, want, what in ((xq, oxq, "X codes"), (xqT, oxqT, "X^T codes"), (wq, owq, "W codes"),
                            (wqT, owqT, "W^T codes"), (gq, ogq, "dY codes"), (gqT, ogqT, "dY^T codes")):
        assert_bytes_equal(host(got), want, what)
    for got, want, what in ((xs, oxs, "X scales"), (xsT, oxsT, "X^T scales"), (ws, ows, "W scales"),
                            (gs, ogs, "dY scales"), (gsT, ogsT, "dY^T scales")):
        assert_scales_equal(host(got), want, what)
    mq, me, mqT, meT = fb.fp8_mx_quantize_1x32(xd)
    omq, ome = oracle.mx_quant_rows(X)
    omqT, omeT = oracle.mx_quant_cols(X)
    for got, want, what in ((mq, omq, "MX codes"), (me, ome, "MX E8M0"), (mqT, omqT, "MX^T codes"),
                            (meT, omeT, "MX^T E8M0")):
        assert_bytes_equal(host(got), want, what)

    # GEMMs, fp32 outputs
    f32 = torch.float32
    y = host(fb.fp8_gemm_fprop(xq, xs, wq, ws, N, D, C, out_dtype=f32))
    dx = host(fb.fp8_gemm_dgrad(gq, gs, wqT, ws, N, D, C, out_dtype=f32))
    dw = host(fb.fp8_gemm_wgrad(gqT, gsT, xqT, xsT, N, D, C, out_dtype=f32))
    Xa = np.abs(oracle.deq_rowgroups(oxq, oxs, C))
    Wa = np.abs(oracle.deq_128x128(owq, ows, D, C))
    Ga = np.abs(oracle.deq_rowgroups(ogq, ogs, D))
    K = ogqT.shape[1]
    GTa = np.abs(oracle.deq_rowgroups(ogqT, ogsT, K))
    XTa = np.abs(oracle.deq_rowgroups(oxqT, oxsT, K))
    for got, want, mag, what in (
            (y, oracle.fprop(oxq, oxs, owq, ows, C), oracle.matmul_f64(Xa, Wa.T), "fprop"),
            (dx, oracle.dgrad(ogq, ogs, owq, ows, D, C), oracle.matmul_f64(Ga, Wa), "dgrad"),
            (dw, oracle.wgrad(ogqT, ogsT, oxqT, oxsT, K), oracle.matmul_f64(GTa, XTa.T), "wgrad")):
        ratio = float(np.max(np.abs(got - want) / np.maximum(mag, 1e-300)))
        assert ratio <= ACC_BOUND, (what, ratio)
        if got.shape[1] >= 16:
            err = oracle.rel_row_error(got, want)
            assert err <= TOL, (what, err)


def _check_gemm(got, want, mag, what):
    ratio = float(np.max(np.abs(got - want) / np.maximum(mag, 1e-300))) if got.size else 0.0
    assert ratio <= ACC_BOUND, (what, ratio)
    if got.ndim == 2 and got.shape[1] >= 16:
        err = oracle.rel_row_error(got, want)
        assert err <= TOL, (what, err)


@pytest.mark.parametrize("N,D,C", SHAPES)
def test_random_shape_mx_gemms(N, D, C):
    """The MXFP8 GEMMs on the same shapes (E8M0 scales on the scaled MFMA)."""
    banner(f"random shape MX N={N} D={D} C={C}")
    rng = np.random.default_rng(N * 7919 + D * 31 + C)
    X = _data(rng, (N, C))
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    dY = (_data(rng, (N, D)) * 1e-3).astype(np.float32)
    xq, xe, xqT, xeT = fb.fp8_mx_quantize_1x32(dev_strided(X))
    wq, we, wqT, weT = fb.fp8_mx_quantize_1x32(dev_strided(W))
    gq, ge, gqT, geT = fb.fp8_mx_quantize_1x32(dev_strided(dY))
    f32 = torch.float32
    y = host(fb.fp8_mx_gemm_fprop(xq, xe, wq, we, N, D, C, out_dtype=f32))
    dx = host(fb.fp8_mx_gemm_dgrad(gq, ge, wqT, weT, N, D, C, out_dtype=f32))
    dw = host(fb.fp8_mx_gemm_wgrad(gqT, geT, xqT, xeT, N, D, C, out_dtype=f32))
    o = {k: oracle.mx_quant_rows(v) for k, v in (("x", X), ("w", W), ("g", dY))}
    oT = {k: oracle.mx_quant_cols(v) for k, v in (("x", X), ("w", W), ("g", dY))}
    a = lambda q, e, k: np.abs(oracle.deq_mx(q, e, k))
    _check_gemm(y, oracle.mx_gemm(*o["x"], *o["w"], C), oracle.matmul_f64(a(*o["x"], C), a(*o["w"], C).T), "mx fprop")
    _check_gemm(dx, oracle.mx_gemm(*o["g"], *oT["w"], D),
                oracle.matmul_f64(a(*o["g"], D), a(*oT["w"], D).T), "mx dgrad")
    _check_gemm(dw, oracle.mx_gemm(*oT["g"], *oT["x"], N),
                oracle.matmul_f64(a(*oT["g"], N), a(*oT["x"], N).T), "mx wgrad")


def _routing(seed: int):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 13))
    sizes = [int(rng.choice([0, 1, 127, 128, 129])) if rng.random() < 0.4 else int(rng.integers(0, 300))
             for _ in range(E)]
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    H = int(rng.choice(EDGES)) if rng.random() < 0.5 else int(rng.integers(1, 300))
    Dn = int(rng.choice([128, 256]))
    return offs, H, Dn


@pytest.mark.parametrize("seed", range(6))
def test_random_grouped_layer(seed):
    """Grouped (MoE) quantization and GEMMs on random routings: 1 to 12
    experts, empty, one-row and 128-boundary experts, ragged hidden sizes;
    the token-axis codes and scales bit for bit, every expert's GEMMs
    against the oracle on that expert's rows."""
    offs, H, Dn = _routing(seed)
    E, R = len(offs) - 1, int(offs[-1])
    banner(f"random grouped layer seed={seed} E={E} rows={R} H={H} Dn={Dn}")
    if R == 0:
        pytest.skip("routing with no rows")
    rng = np.random.default_rng(1000 + seed)
    X = _data(rng, (R, H))
    dY = (_data(rng, (R, Dn)) * 1e-3).astype(np.float32)
    Ws = (rng.standard_normal((E, Dn, H)) * 0.02).astype(np.float32)
    od = torch.from_numpy(offs).to("cuda")
    xqT, xsT, xq, xs = fb.fp8_quantize_transposed_grouped(dev_strided(X), od, rowwise=True)
    gqT, gsT, gq, gs = fb.fp8_quantize_transposed_grouped(dev_strided(dY), od, rowwise=True)
    oqT, osT = oracle.quant_colwise(X, offs)
    P = oqT.shape[1]
    assert_bytes_equal(host(xqT)[:, :P], oqT, "grouped X^T codes")
    assert_scales_equal(host(xsT)[:, :P // 128], osT, "grouped X^T scales")
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(dev_strided(Ws.reshape(E * Dn, H)))
    f32 = torch.float32
    nbs = Dn // 128
    y = host(fb.fp8_gemm_fprop_grouped(xq, xs, wq, Dn * wq.stride(0), ws, nbs * ws.stride(0), od, R, Dn, H,
                                       out_dtype=f32))
    dx = host(fb.fp8_gemm_dgrad_grouped(gq, gs, wqT, Dn, ws, nbs * ws.stride(0), od, R, Dn, H, out_dtype=f32))
    dw = host(fb.fp8_gemm_wgrad_grouped(gqT, gsT, xqT, xsT, od, R, Dn, H, out_dtype=f32))
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if a == b:
            assert np.all(dw[e] == 0), f"empty expert {e}"
            continue
        oxq, oxs = oracle.quant_1x128(X[a:b])
        owq, ows, _ = oracle.quant_128x128(Ws[e], with_transpose=False)
        ogq, ogs = oracle.quant_1x128(dY[a:b])
        ogqT, ogsT = oracle.quant_colwise(dY[a:b])
        oxqT, oxsT = oracle.quant_colwise(X[a:b])
        K = ogqT.shape[1]
        Xa = np.abs(oracle.deq_rowgroups(oxq, oxs, H))
        Wa = np.abs(oracle.deq_128x128(owq, ows, Dn, H))
        Ga = np.abs(oracle.deq_rowgroups(ogq, ogs, Dn))
        GTa = np.abs(oracle.deq_rowgroups(ogqT, ogsT, K))
        XTa = np.abs(oracle.deq_rowgroups(oxqT, oxsT, K))
        _check_gemm(y[a:b], oracle.fprop(oxq, oxs, owq, ows, H), oracle.matmul_f64(Xa, Wa.T), f"e{e} fprop")
        _check_gemm(dx[a:b], oracle.dgrad(ogq, ogs, owq, ows, Dn, H), oracle.matmul_f64(Ga, Wa), f"e{e} dgrad")
        _check_gemm(dw[e], oracle.wgrad(ogqT, ogsT, oxqT, oxsT, K), oracle.matmul_f64(GTa, XTa.T), f"e{e} wgrad")


@pytest.mark.parametrize("N,D,C", SHAPES)
def test_random_shape_variants(N, D, C):
    """The variants on the same shapes: power-of-two scales (codes, scales
    and E8M0 bytes bit for bit), the token-axis requantization of the saved
    1x128 copy (bit for bit), and, for at most 64 tokens, FProp on the packed
    decode weight (bit for bit the row-major FProp, both recipes)."""
    banner(f"random shape variants N={N} D={D} C={C}")
    rng = np.random.default_rng(N * 104729 + D * 7 + C)
    X = _data(rng, (N, C))
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    xd, wd = dev_strided(X), dev_strided(W)
    # power-of-two scales
    pq, ps, pe = fb.fp8_quantize_act_1x128_pow2(xd)
    oq, os_ = oracle.quant_1x128(X, pow2=True)
    assert_bytes_equal(host(pq), oq, "pow2 codes")
    assert_scales_equal(host(ps), os_, "pow2 scales")
    assert_bytes_equal(host(pe), np.repeat(oracle.e8m0_of_pow2(os_), 4, axis=1), "pow2 E8M0")
    pqT, psT, _, _, _, _ = fb.fp8_quantize_transposed_pow2(xd, rowwise=False, e8=False)
    oqT, osT = oracle.quant_colwise(X, pow2=True)
    assert_bytes_equal(host(pqT), oqT, "pow2 token-axis codes")
    assert_scales_equal(host(psT), osT, "pow2 token-axis scales")
    # requantization of the saved row-wise copy
    xq, xs = fb.fp8_quantize_act_1x128(xd)
    rqT, rsT = fb.fp8_requantize_transposed(xq, xs, C)
    ox, oxs = oracle.quant_1x128(X)
    orqT, orsT = oracle.requant_colwise(ox, oxs, C)
    assert_bytes_equal(host(rqT), orqT, "requantized codes")
    assert_scales_equal(host(rsT), orsT, "requantized scales")
    # rollout decode on the packed weight
    if N <= 64:
        wq, ws, _ = fb.fp8_quantize_weight_128x128(wd, transpose=False)
        wp, _ = fb.fp8_pack_decode_weight(wq, D, C)
        mxq, mxe, _, _ = fb.fp8_mx_quantize_1x32(xd, colwise=False)
        mwq, mwe, _, _ = fb.fp8_mx_quantize_1x32(wd, colwise=False)
        mwp, mwep = fb.fp8_pack_decode_weight(mwq, D, C, we=mwe)
        for dt in (torch.float32, torch.bfloat16):
            assert torch.equal(fb.fp8_gemm_fprop_decode(xq, xs, wp, ws, N, D, C, out_dtype=dt),
                               fb.fp8_gemm_fprop(xq, xs, wq, ws, N, D, C, out_dtype=dt)), ("decode", dt)
            assert torch.equal(fb.fp8_mx_gemm_fprop_decode(mxq, mxe, mwp, mwep, N, D, C, out_dtype=dt),
                               fb.fp8_mx_gemm_fprop(mxq, mxe, mwq, mwe, N, D, C, out_dtype=dt)), ("mx decode", dt)


def _bits(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> host uint16 bits."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("N,D,C", SHAPES)
def test_random_shape_fused_producers(N, D, C):
    """RMSNorm + 1x128 (bf16 and fp32 rows, bf16 weights) on [N x C] and
    SiLU(gate)*up + 1x128 on [N x D] (gate and up views of one matrix):
    codes, scales, the bf16 activation and RMSNorm's r bit for bit."""
    banner(f"random fused producers N={N} D={D} C={C}")
    rng = np.random.default_rng(N * 7919 + D * 104729 + C)
    X = _data(rng, (N, C))
    w = oracle.bf16_rne((1 + 0.1 * rng.standard_normal(C)).astype(np.float32))
    wd = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to("cuda")
    for x, kind in ((oracle.bf16_rne(X), "bf16"), (X, "fp32")):
        q, s, r, y = fb.fp8_rmsnorm_quantize_1x128(dev_strided(x), wd, 1e-6, rstd=True, y=True)
        oq, os_, orr, oy = oracle.rmsnorm_quant_1x128(x, w, 1e-6)
        assert_scales_equal(host(r), orr, f"rmsnorm {kind} rstd")
        assert_bytes_equal(_bits(y), oy, f"rmsnorm {kind} y")
        assert_bytes_equal(host(q), oq, f"rmsnorm {kind} codes")
        assert_scales_equal(host(s), os_, f"rmsnorm {kind} scales")
    gate = oracle.bf16_rne((2.0 * rng.standard_normal((N, D))).astype(np.float32))
    up = oracle.bf16_rne(_data(rng, (N, D)))
    pad = (-D) % 8
    H = np.zeros((N, 2 * (D + pad)), np.uint16)
    H[:, :D] = gate
    H[:, D + pad:2 * D + pad] = up
    Hd = torch.from_numpy(H.view(np.int16)).view(torch.bfloat16).to("cuda")
    q, s, a = fb.fp8_silu_mul_quantize_1x128(Hd[:, :D], Hd[:, D + pad:2 * D + pad], a=True)
    oq, os_, oa = oracle.silu_mul_quant_1x128(gate, up)
    assert_bytes_equal(_bits(a), oa, "silu*up activation")
    assert_bytes_equal(host(q), oq, "silu*up codes")
    assert_scales_equal(host(s), os_, "silu*up scales")
