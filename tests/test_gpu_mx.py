"""GPU parity of the MXFP8 path (Miles blog, MXFP8 paragraphs) against the
oracle: E4M3 codes and E8M0 bytes bit-exact in both orientations, MX GEMMs
within the 2e-3 row-norm tolerance, on the decode-shaped MX workload and on
ragged shapes."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_02_amd as fb
import oracle
from block_scaled_fp8_02_amd import workloads as wl
from gpu_util import TOL, assert_bytes_equal, assert_scales_equal, banner, dev, dev_strided, host

pytestmark = pytest.mark.gpu


def check_mx_quant(x_host):
    q, e, qT, eT = fb.fp8_mx_quantize_1x32(dev_strided(x_host))
    oq, oe = oracle.mx_quant_rows(x_host)
    oqT, oeT = oracle.mx_quant_cols(x_host)
    assert_bytes_equal(host(q), oq, "mx row codes")
    assert_bytes_equal(host(e), oe, "mx row scales")
    assert_bytes_equal(host(qT), oqT, "mx col codes")
    assert_bytes_equal(host(eT), oeT, "mx col scales")


@pytest.mark.parametrize("shape", [(1, 1), (3, 300), (129, 257), (64, 4096), (300, 33)])
def test_mx_quant_ragged(shape):
    banner(f"mx quant {shape}")
    rng = np.random.default_rng(sum(shape) + 1)
    x = (rng.standard_normal(shape) * np.exp(rng.uniform(-20, 20, shape))).astype(np.float32)
    x[0, :min(32, shape[1])] = 0.0
    check_mx_quant(x)
    check_mx_quant(wl.f32_to_bf16_bits(x))


@pytest.mark.parametrize("shape", [(1, 1), (3, 300), (129, 257), (64, 4096), (300, 33), (2, 24576)])
def test_mx_quant_rowwise_only(shape):
    """The row-wise copy alone (the rollout's activation: no transposed
    codes) runs a kernel of its own; its codes and E8M0 bytes equal the
    oracle's and the two-orientation kernel's, with 4-byte-aligned scale rows
    (word stores) and with odd ones (byte stores)."""
    banner(f"mx quant row-wise only {shape}")
    rows, cols = shape
    rng = np.random.default_rng(rows * 31 + cols)
    x = (rng.standard_normal(shape) * np.exp(rng.uniform(-20, 20, shape))).astype(np.float32)
    x[0, :min(32, cols)] = 0.0
    for xin in (x, wl.f32_to_bf16_bits(x)):
        xd = dev_strided(xin)
        q, e, qT, eT = fb.fp8_mx_quantize_1x32(xd, colwise=False)
        assert qT is None and eT is None
        oq, oe = oracle.mx_quant_rows(xin)
        assert_bytes_equal(host(q), oq, "mx row-wise-only codes")
        assert_bytes_equal(host(e), oe, "mx row-wise-only scales")
        q2, e2, _, _ = fb.fp8_mx_quantize_1x32(xd)
        assert torch.equal(q, q2) and torch.equal(e, e2), "row-wise-only != two-orientation row-wise copy"
        kb = -(-cols // 128) * 4
        q3 = torch.empty((rows, -(-cols // 128) * 128), dtype=torch.uint8, device="cuda")
        e3 = torch.empty((rows, kb + 1), dtype=torch.uint8, device="cuda")[:, :kb]
        fb.fp8_mx_quantize_1x32(xd, colwise=False, q=q3, e=e3)
        assert_bytes_equal(host(q3), oq, "mx row-wise-only codes (odd scale stride)")
        assert_bytes_equal(host(e3), oe, "mx row-wise-only scales (odd scale stride)")


@pytest.mark.parametrize("shape", [(129, 300), (64, 4096)])
def test_mx_quant_odd_scale_strides(shape):
    """E8M0 rows whose stride is not a multiple of 4 bytes: the quantizer
    stores those scales byte by byte (4-byte rows take one word per tile);
    both orientations bit-exact against the oracle."""
    rows, cols = shape
    banner(f"mx quant, odd E8M0 strides {shape}")
    rng = np.random.default_rng(rows + cols)
    x = (rng.standard_normal(shape) * np.exp(rng.uniform(-4, 4, shape))).astype(np.float32)
    kb, kbT = -(-cols // 128) * 4, -(-rows // 128) * 4
    q = torch.empty((rows, -(-cols // 128) * 128), dtype=torch.uint8, device="cuda")
    qT = torch.empty((cols, -(-rows // 128) * 128), dtype=torch.uint8, device="cuda")
    e = torch.empty((rows, kb + 1), dtype=torch.uint8, device="cuda")[:, :kb]
    eT = torch.empty((cols, kbT + 3), dtype=torch.uint8, device="cuda")[:, :kbT]
    fb.fp8_mx_quantize_1x32(dev_strided(x), q=q, e=e, qT=qT, eT=eT)
    oq, oe = oracle.mx_quant_rows(x)
    oqT, oeT = oracle.mx_quant_cols(x)
    assert_bytes_equal(host(q), oq, "mx row codes")
    assert_bytes_equal(host(e), oe, "mx row scales (odd stride)")
    assert_bytes_equal(host(qT), oqT, "mx col codes")
    assert_bytes_equal(host(eT), oeT, "mx col scales (odd stride)")


def test_mx_quant_classes():
    x = np.zeros((64, 256), np.float32)
    x[1] = np.finfo(np.float32).max
    x[2] = np.uint32(1).view(np.float32)
    x[3] = -0.0
    x[4, ::3] = 448.0 * 2.0 ** -130
    x[5] = np.linspace(-3, 3, 256).astype(np.float32)
    check_mx_quant(x)


def test_mx_workload_full():
    """The MXFP8 workload (decode shapes: X [64 x 4096], fused gate+up W
    [24576 x 4096], dY [64 x 24576]): codes and E8M0 bytes of all three
    tensors in both orientations bit for bit, and every output of FProp,
    DGrad (split along K, as the benchmark runs it) and WGrad (K = 64)
    against the oracle."""
    w = wl.mx(0)
    banner("mx workload: quantize X, W, dY in both orientations; FProp/DGrad/WGrad")
    X, W, dY = w["X"], w["W"], w["dY"]
    N, C, D = 64, 4096, 24576
    xq, xe, xqT, xeT = fb.fp8_mx_quantize_1x32(dev(X))
    wq, we, wqT, weT = fb.fp8_mx_quantize_1x32(dev(W))
    gq, ge, gqT, geT = fb.fp8_mx_quantize_1x32(dev(dY))
    y = host(fb.fp8_mx_gemm_fprop(xq, xe, wq, we, N, D, C))
    dx = host(fb.fp8_mx_gemm_dgrad(gq, ge, wqT, weT, N, D, C))
    dw = host(fb.fp8_mx_gemm_wgrad(gqT, geT, xqT, xeT, N, D, C))
    banner("mx workload: oracle")
    ora = {}
    for name, t, got in (("X", X, (xq, xe, xqT, xeT)), ("W", W, (wq, we, wqT, weT)),
                         ("dY", dY, (gq, ge, gqT, geT))):
        oq, oe = oracle.mx_quant_rows(t)
        oqT, oeT = oracle.mx_quant_cols(t)
        for g, o, what in zip(got, (oq, oe, oqT, oeT), ("row codes", "row scales", "col codes", "col scales")):
            assert_bytes_equal(host(g), o, f"mx {name} {what}")
        ora[name] = (oq, oe, oqT, oeT)
    (oxq, oxe, oxqT, oxeT), (owq, owe, owqT, oweT), (ogq, oge, ogqT, ogeT) = ora["X"], ora["W"], ora["dY"]
    for got, ref, name in ((y, oracle.mx_gemm(oxq, oxe, owq, owe, C), "fprop"),
                           (dx, oracle.mx_gemm(ogq, oge, owqT, oweT, D), "dgrad"),
                           (dw, oracle.mx_gemm(ogqT, ogeT, oxqT, oxeT, N), "wgrad")):
        err = oracle.rel_row_error(got, ref)
        banner(f"mx {name} err (full) {err:.3e}")
        assert err <= TOL, (name, err)


def test_blockscaled_path_on_mx_workload_full():
    """The 1x128 / 128x128 path on the same tensors as the MXFP8 workload:
    quantizer outputs bit for bit (X row-wise and token-axis, W with its
    transposed codes, dY row-wise along D and token-axis) and every output
    of FProp, DGrad (64 x 4096 with K = 24576, split along K) and WGrad
    (24576 x 4096 with K = 64, one partial token group) against the oracle,
    in the launch configurations the benchmark times."""
    w = wl.mx(0)
    X, W, dY = w["X"], w["W"], w["dY"]
    N, C, D = 64, 4096, 24576
    banner("1x128 path on the mx workload: quantize + FProp/DGrad/WGrad")
    xqT, xsT, xq, xs = fb.fp8_quantize_transposed(dev(X), rowwise=True)
    gqT, gsT, gq, gs = fb.fp8_quantize_transposed(dev(dY), rowwise=True)
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(dev(W))
    y = host(fb.fp8_gemm_fprop(xq, xs, wq, ws, N, D, C))
    dx = host(fb.fp8_gemm_dgrad(gq, gs, wqT, ws, N, D, C))
    dw = host(fb.fp8_gemm_wgrad(gqT, gsT, xqT, xsT, N, D, C))
    banner("1x128 path on the mx workload: oracle")
    oxq, oxs = oracle.quant_1x128(X)
    oxqT, oxsT = oracle.quant_colwise(X)
    ogq, ogs = oracle.quant_1x128(dY)
    ogqT, ogsT = oracle.quant_colwise(dY)
    owq, ows, owqT = oracle.quant_128x128(W)
    for g, o, what in ((xq, oxq, "X codes"), (xqT, oxqT, "X token-axis codes"), (gq, ogq, "dY codes"),
                       (gqT, ogqT, "dY token-axis codes"), (wq, owq, "W codes"), (wqT, owqT, "W^T codes")):
        assert_bytes_equal(host(g), o, what)
    for g, o, what in ((xs, oxs, "X scales"), (xsT, oxsT, "X token-axis scales"), (gs, ogs, "dY scales"),
                       (gsT, ogsT, "dY token-axis scales"), (ws, ows, "W scales")):
        assert_scales_equal(host(g), o, what)
    for got, ref, name in ((y, oracle.fprop(oxq, oxs, owq, ows, C), "fprop"),
                           (dx, oracle.dgrad(ogq, ogs, owq, ows, D, C), "dgrad (K split)"),
                           (dw, oracle.wgrad(ogqT, ogsT, oxqT, oxsT, N), "wgrad (K = 64)")):
        err = oracle.rel_row_error(got, ref)
        banner(f"1x128 {name} err (full) {err:.3e}")
        assert err <= TOL, (name, err)


@pytest.mark.parametrize("N,D,C", [(1, 16, 32), (3, 130, 300), (200, 300, 260), (257, 384, 1024)])
def test_mx_gemm_ragged(N, D, C):
    rng = np.random.default_rng(N + D + C)
    X = (rng.standard_normal((N, C)) * np.exp(rng.uniform(-3, 3, (N, C)))).astype(np.float32)
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    dY = (rng.standard_normal((N, D)) * 1e-3).astype(np.float32)
    xq, xe, xqT, xeT = fb.fp8_mx_quantize_1x32(dev_strided(X))
    wq, we, wqT, weT = fb.fp8_mx_quantize_1x32(dev_strided(W))
    gq, ge, gqT, geT = fb.fp8_mx_quantize_1x32(dev_strided(dY))
    y = host(fb.fp8_mx_gemm_fprop(xq, xe, wq, we, N, D, C, out_dtype=torch.float32))
    dx = host(fb.fp8_mx_gemm_dgrad(gq, ge, wqT, weT, N, D, C, out_dtype=torch.float32))
    dw = host(fb.fp8_mx_gemm_wgrad(gqT, geT, xqT, xeT, N, D, C, out_dtype=torch.float32))
    oxq, oxe = oracle.mx_quant_rows(X)
    owq, owe = oracle.mx_quant_rows(W)
    owqT, oweT = oracle.mx_quant_cols(W)
    ogq, oge = oracle.mx_quant_rows(dY)
    ogqT, ogeT = oracle.mx_quant_cols(dY)
    oxqT, oxeT = oracle.mx_quant_cols(X)
    mag = {"fprop": oracle.matmul_f64(np.abs(oracle.deq_mx(oxq, oxe, C)), np.abs(oracle.deq_mx(owq, owe, C)).T),
           "dgrad": oracle.matmul_f64(np.abs(oracle.deq_mx(ogq, oge, D)), np.abs(oracle.deq_mx(owqT, oweT, D)).T),
           "wgrad": oracle.matmul_f64(np.abs(oracle.deq_mx(ogqT, ogeT, N)), np.abs(oracle.deq_mx(oxqT, oxeT, N)).T)}
    for got, ref, name in ((y, oracle.mx_gemm(oxq, oxe, owq, owe, C), "fprop"),
                           (dx, oracle.mx_gemm(ogq, oge, owqT, oweT, D), "dgrad"),
                           (dw, oracle.mx_gemm(ogqT, ogeT, oxqT, oxeT, N), "wgrad")):
        err = oracle.rel_row_error(got, ref)
        ratio = float(np.max(np.abs(got - ref) / np.maximum(mag[name], 1e-300)))
        banner(f"mx ragged {name} N={N} D={D} C={C}: {err:.3e}, |err|/sum|ab| {ratio:.3e}")
        assert err <= TOL
        assert ratio <= 2.0 ** -12          # fp8 MFMA dot-product accumulation scale


def test_mx_forward_is_batch_invariant():
    """MX FProp rows do not depend on how many rows are in the call: the
    decode tiles (64 x 128 for this weight, 64 x 16 for a narrow one) give
    the 256 x 256 training tile's rows bit for bit."""
    w = wl.mx(0)
    rng = wl.rng_for(11)
    X = wl.f32_to_bf16_bits(wl.normal(rng, (512, 4096), 1.0))
    banner("mx batch invariance 1/17/64 vs 512 rows")
    wq, we, _, _ = fb.fp8_mx_quantize_1x32(dev(w["W"]), colwise=False)
    xq, xe, _, _ = fb.fp8_mx_quantize_1x32(dev(X), colwise=False)
    for D in (24576, 4000):
        y_big = fb.fp8_mx_gemm_fprop(xq, xe, wq[:D], we[:D], 512, D, 4096)
        for m in (1, 17, 64):
            xqm, xem, _, _ = fb.fp8_mx_quantize_1x32(dev(X[:m]), colwise=False)
            ym = fb.fp8_mx_gemm_fprop(xqm, xem, wq[:D], we[:D], m, D, 4096)
            assert torch.equal(ym, y_big[:m]), (D, m)


@pytest.mark.parametrize("M,D,C", [(1, 12289, 1), (37, 12289, 300), (64, 12300, 1100),
                                   (64, 12193, 4099)])
def test_mx_decode_rows_kernel_ragged(M, D, C):
    """Decode-shaped MX FProp (weight-streaming decode kernel): oracle parity
    at ragged shapes, and the 80-row call's rows bit for bit."""
    banner(f"mx decode rows kernel M={M} D={D} C={C}")
    rng = np.random.default_rng(M * 3 + D + C)
    X = (rng.standard_normal((80, C)) * np.exp(rng.uniform(-3, 3, (80, C)))).astype(np.float32)
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    xq, xe, _, _ = fb.fp8_mx_quantize_1x32(dev_strided(X), colwise=False)
    wq, we, _, _ = fb.fp8_mx_quantize_1x32(dev_strided(W), colwise=False)
    y = host(fb.fp8_mx_gemm_fprop(xq[:M], xe[:M], wq, we, M, D, C, out_dtype=torch.float32))
    oxq, oxe = oracle.mx_quant_rows(X[:M])
    owq, owe = oracle.mx_quant_rows(W)
    mag = oracle.matmul_f64(np.abs(oracle.deq_mx(oxq, oxe, C)), np.abs(oracle.deq_mx(owq, owe, C)).T)
    ref = oracle.mx_gemm(oxq, oxe, owq, owe, C)
    err = oracle.rel_row_error(y, ref)
    ratio = float(np.max(np.abs(y - ref) / np.maximum(mag, 1e-300)))
    banner(f"mx decode rows: {err:.3e}, |err|/sum|ab| {ratio:.3e}")
    assert err <= TOL
    assert ratio <= 2.0 ** -12
    for dt in (torch.float32, torch.bfloat16):
        y_big = fb.fp8_mx_gemm_fprop(xq, xe, wq, we, 80, D, C, out_dtype=dt)
        y_m = fb.fp8_mx_gemm_fprop(xq[:M], xe[:M], wq, we, M, D, C, out_dtype=dt)
        assert torch.equal(y_m, y_big[:M]), dt


def packed_scale_words_ref(we_host, D, C):
    """Packed MX scale words with numpy: word (group, K block, r) holds row
    16 group + r's four E8M0 bytes of that K block (127s past D)."""
    KB, R = (C + 127) // 128, (D + 15) // 16 * 16
    b = np.full((R, KB * 4), 127, np.uint8)
    b[:D] = we_host[:D, :KB * 4]
    words = b.reshape(R, KB, 4).copy().view(np.int32).reshape(R, KB)     # little-endian words
    return np.ascontiguousarray(words.reshape(R // 16, 16, KB).transpose(0, 2, 1)).reshape(R, KB)


@pytest.mark.parametrize("M,D,C", [(1, 1, 1), (5, 17, 130), (37, 12289, 300), (64, 12300, 1100),
                                   (64, 12193, 4099), (64, 24576, 4096)])
def test_mx_decode_packed_matches_fprop(M, D, C):
    """MX FProp on the packed weight and scale words: the packing checked
    byte for byte, the output bit for bit the row-major MX FProp."""
    banner(f"mx decode packed M={M} D={D} C={C}")
    rng = np.random.default_rng(M + 5 * D + C)
    X = (rng.standard_normal((M, C)) * np.exp(rng.uniform(-3, 3, (M, C)))).astype(np.float32)
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    xq, xe, _, _ = fb.fp8_mx_quantize_1x32(dev_strided(X), colwise=False)
    wq, we, _, _ = fb.fp8_mx_quantize_1x32(dev_strided(W), colwise=False)
    wp, wep = fb.fp8_pack_decode_weight(wq, D, C, we=we)
    np.testing.assert_array_equal(host(wep), packed_scale_words_ref(host(we), D, C))
    for dt in (torch.float32, torch.bfloat16):
        y_row = fb.fp8_mx_gemm_fprop(xq, xe, wq, we, M, D, C, out_dtype=dt)
        y_dec = fb.fp8_mx_gemm_fprop_decode(xq, xe, wp, wep, M, D, C, out_dtype=dt)
        assert torch.equal(y_dec, y_row), dt
