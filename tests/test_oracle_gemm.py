"""Pins for the oracle's block-scaled GEMMs (CPU only).

* Exact rational brute force (fractions.Fraction over the decoded codes and
  the fp32 scales) on two-row problems with one or two 128-wide blocks on
  the other axes, for FProp, DGrad and WGrad, with scales that differ from block to block so a wrong scale index
  or a transposed operand fails.  The oracle's fp64 sums must sit within the
  standard fp64 summation bound of the exact values.
* The lossless case reduces to a plain fp64 matrix product of the original
  inputs (numpy matmul).
* DGrad read through the transposed weight copy is bit-identical to DGrad
  read from the stored orientation (the weight scales are symmetric, so the
  transpose changes no value: Jet-RL notes, DGrad/WGrad paragraph).
* WGrad equals the sum over tokens of per-token outer products.
* The shape algebra of the three GEMMs (Jet-RL notes, "Quantization of
  linear layers": Y is N x D, dW is D x C, dX is N x C).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

TABLE = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
    .to(torch.float64).numpy()
FRAC = [Fraction(float(v)) if np.isfinite(v) else None for v in TABLE]


def deq_exact_rows(q, s, K, group=128):
    return [[FRAC[q[r, k]] * Fraction(float(s[r, k // group])) for k in range(K)]
            for r in range(q.shape[0])]


def deq_exact_blocks(q, s, D, C):
    return [[FRAC[q[d, c]] * Fraction(float(s[d // 128, c // 128])) for c in range(C)]
            for d in range(D)]


def exact_mm(A, B_rows):
    """out[i][j] = sum_k A[i][k] * B_rows[j][k] exactly."""
    return [[sum((a * b for a, b in zip(Ai, Bj)), Fraction(0)) for Bj in B_rows] for Ai in A]


def check_close_to_exact(y, exact, A, B_rows):
    K = len(A[0])
    for i in range(len(A)):
        for j in range(len(B_rows)):
            mag = sum(abs(float(a) * float(b)) for a, b in zip(A[i], B_rows[j]))
            err = abs(Fraction(float(y[i, j])) - exact[i][j])
            assert float(err) <= K * 2.0 ** -53 * mag * 1.01 + 1e-300, (i, j)


def graded(rng, shape, col_blocks=True):
    """Random values whose magnitude changes by block, so every scale differs."""
    x = rng.standard_normal(shape)
    r = np.exp(rng.uniform(-6, 6, size=(shape[0] // 1, (shape[1] + 127) // 128)))
    return (x * np.repeat(r, 128, axis=1)[:, :shape[1]]).astype(np.float32)


@pytest.mark.parametrize("C", [128, 256])
def test_fprop_exact_brute_force(C):
    rng = np.random.default_rng(20 + C)
    X = graded(rng, (2, C))
    W = (rng.standard_normal((256, C)) * np.exp(rng.uniform(-4, 4))).astype(np.float32)
    W[:, 128:] *= np.float32(7.0)
    W[128:, :] *= np.float32(0.01)
    xq, xs = oracle.quant_1x128(X)
    wq, ws, _ = oracle.quant_128x128(W, with_transpose=False)
    y = oracle.fprop(xq, xs, wq, ws, C)
    assert y.shape == (2, 256)
    A = deq_exact_rows(xq, xs, C)
    B = deq_exact_blocks(wq, ws, 256, C)
    check_close_to_exact(y, exact_mm(A, B), A, B)


@pytest.mark.parametrize("D", [128, 256])
def test_dgrad_exact_brute_force(D):
    rng = np.random.default_rng(30 + D)
    C = 256
    G = graded(rng, (2, D))
    W = (rng.standard_normal((D, C)) * 0.02).astype(np.float32)
    W[128:] *= np.float32(0.01)
    W[:, 128:] *= np.float32(9.0)
    gq, gs = oracle.quant_1x128(G)
    wq, ws, wqT = oracle.quant_128x128(W)
    y = oracle.dgrad(gq, gs, wq, ws, D, C)
    assert y.shape == (2, C)
    A = deq_exact_rows(gq, gs, D)
    Wd = deq_exact_blocks(wq, ws, D, C)
    B_rows = [[Wd[d][c] for d in range(D)] for c in range(C)]   # W^T rows
    check_close_to_exact(y, exact_mm(A, B_rows), A, B_rows)
    assert np.array_equal(oracle.dgrad_from_qT(gq, gs, wqT, ws, D, C), y)


@pytest.mark.parametrize("N", [128, 256])
def test_wgrad_exact_brute_force(N):
    rng = np.random.default_rng(40 + N)
    D, C = 2, 130
    G = (rng.standard_normal((N, D)) * 1e-3).astype(np.float32)
    X = rng.standard_normal((N, C)).astype(np.float32)
    G[128:] *= np.float32(30.0)
    X[128:] *= np.float32(0.1)
    gqT, gsT = oracle.quant_colwise(G)
    xqT, xsT = oracle.quant_colwise(X)
    y = oracle.wgrad(gqT, gsT, xqT, xsT, N)
    assert y.shape == (D, C)
    A = deq_exact_rows(gqT, gsT, N)
    B = deq_exact_rows(xqT, xsT, N)
    check_close_to_exact(y, exact_mm(A, B), A, B)


def test_lossless_case_is_plain_fp64_matmul():
    rng = np.random.default_rng(50)
    N, C, D = 64, 384, 256
    # operands built from E4M3 values times power-of-two scales with each
    # group/tile reaching 448*2^k, so quantization is exact
    codes_x = rng.integers(0, 0x7E, size=(N, C)) | (rng.integers(0, 2, (N, C)) << 7)
    codes_x[:, ::128] = 0x7E
    kx = rng.integers(-8, 8, size=(N, C // 128))
    X = (TABLE[codes_x] * np.repeat(np.ldexp(1.0, kx), 128, axis=1)).astype(np.float32)
    codes_w = rng.integers(0, 0x7E, size=(D, C)) | (rng.integers(0, 2, (D, C)) << 7)
    codes_w[::128, ::128] = 0x7E
    kw = rng.integers(-12, -4, size=(D // 128, C // 128))
    W = (TABLE[codes_w] * np.kron(np.ldexp(1.0, kw), np.ones((128, 128)))).astype(np.float32)
    xq, xs = oracle.quant_1x128(X)
    wq, ws, wqT = oracle.quant_128x128(W)
    y = oracle.fprop(xq, xs, wq, ws, C)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    G = X[:, :D].copy()
    gq, gs = oracle.quant_1x128(G)
    dx = oracle.dgrad(gq, gs, wq, ws, D, C)
    ref2 = G.astype(np.float64) @ W.astype(np.float64)
    assert np.max(np.abs(dx - ref2)) <= 1e-12 * np.max(np.abs(ref2))


def test_wgrad_is_sum_of_outer_products():
    rng = np.random.default_rng(60)
    N, D, C = 300, 48, 40
    G = (rng.standard_normal((N, D)) * 1e-3).astype(np.float32)
    X = rng.standard_normal((N, C)).astype(np.float32)
    gqT, gsT = oracle.quant_colwise(G)
    xqT, xsT = oracle.quant_colwise(X)
    y = oracle.wgrad(gqT, gsT, xqT, xsT, gqT.shape[1])
    Gd = oracle.deq_rowgroups(gqT, gsT, gqT.shape[1])[:, :N]      # D x N
    Xd = oracle.deq_rowgroups(xqT, xsT, xqT.shape[1])[:, :N]      # C x N
    ref = np.zeros((D, C))
    for n in range(N):
        ref += np.outer(Gd[:, n], Xd[:, n])
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_padding_contributes_nothing():
    rng = np.random.default_rng(70)
    X = rng.standard_normal((5, 200)).astype(np.float32)
    W = rng.standard_normal((7, 200)).astype(np.float32)
    xq, xs = oracle.quant_1x128(X)
    wq, ws, _ = oracle.quant_128x128(W, with_transpose=False)
    y200 = oracle.fprop(xq, xs, wq, ws, 200)
    y256 = oracle.fprop(xq, xs, wq, ws, 256)                      # reads the zero padding
    assert np.array_equal(y200, y256)


def test_shape_algebra():
    rng = np.random.default_rng(80)
    N, C, D = 8, 256, 128
    X = rng.standard_normal((N, C)).astype(np.float32)
    W = rng.standard_normal((D, C)).astype(np.float32)
    G = rng.standard_normal((N, D)).astype(np.float32)
    xq, xs = oracle.quant_1x128(X)
    wq, ws, _ = oracle.quant_128x128(W)
    gq, gs = oracle.quant_1x128(G)
    gqT, gsT = oracle.quant_colwise(G)
    xqT, xsT = oracle.quant_colwise(X)
    assert oracle.fprop(xq, xs, wq, ws, C).shape == (N, D)
    assert oracle.dgrad(gq, gs, wq, ws, D, C).shape == (N, C)
    assert oracle.wgrad(gqT, gsT, xqT, xsT, 128).shape == (D, C)


def test_rel_row_error_metric():
    ref = np.array([[3.0, 4.0], [0.0, 0.0]])
    assert oracle.rel_row_error(ref, ref) == 0.0
    assert oracle.rel_row_error(ref + [[0.5, 0.0], [0.0, 0.0]], ref) == pytest.approx(0.1)
    assert oracle.rel_row_error(ref + [[0.0, 0.0], [1e-30, 0.0]], ref) == float("inf")
