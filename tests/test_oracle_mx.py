"""Pins for the oracle's MXFP8 path (CPU only).

Miles MXFP8/NVFP4 blog, MXFP8 paragraphs: 32 consecutive E4M3 values share
one E8M0 power-of-two scale, rounded up so the block maximum is not
clipped; row-wise 1x32 and column-wise 32x1 copies are numerically
different and each is quantized from the full-precision data.

Pins: the exponent is the smallest one that does not clip (checked with
plain Python float arithmetic), no scaled element exceeds 448, a brute-force
encode of tiny blocks, the column-wise copy is the row-wise quantization of
the transpose (and in general not the transpose of the row-wise copy), a
lossless power-of-two construction, and exact rational brute force for the
MX GEMM.
"""
from fractions import Fraction
import json
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")
TABLE = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
    .to(torch.float64).numpy()
FINITE = np.array([c for c in range(128) if c != 0x7F])


def brute_code_f64(y: float) -> int:
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0
    a = abs(y)
    if a >= 448.0:
        return 0x7E | sign
    d = np.abs(TABLE[FINITE] - a)
    cands = FINITE[d == d.min()]
    c = int(cands[0]) if len(cands) == 1 else int(cands[0] if cands[0] % 2 == 0 else cands[1])
    return c | sign


def test_block_size_from_page():
    g = json.load(open(GOLDEN))
    x = np.ones((2, 256), np.float32)
    q, e = oracle.mx_quant_rows(x)
    assert e.shape[1] == 256 // g["mx_block"]["size"]


def test_exponent_is_minimal_non_clipping():
    rng = np.random.default_rng(90)
    vals = np.concatenate([
        np.exp(rng.uniform(-100, 88, 20000)),
        [448.0 * 2.0 ** k for k in range(-140, 120)],
        [np.nextafter(448.0 * 2.0 ** k, 0) for k in range(-120, 120)],
        [np.nextafter(448.0 * 2.0 ** k, np.inf) for k in range(-120, 120)],
        [2.0 ** -149, 2.0 ** -126, 1.0, np.finfo(np.float32).max],
    ]).astype(np.float32)
    for a in vals:
        a = float(a)
        k = oracle.mx_exponent(a)
        assert -127 <= k <= 127
        assert a <= 448.0 * 2.0 ** k
        if k > -127:
            assert a > 448.0 * 2.0 ** (k - 1)
    assert oracle.mx_exponent(0.0) == -127


def test_rows_brute_force_and_no_clipping():
    rng = np.random.default_rng(91)
    x = (rng.standard_normal((6, 100)) * np.exp(rng.uniform(-30, 30, (6, 1)))).astype(np.float32)
    x[0, :32] = 0.0
    q, e = oracle.mx_quant_rows(x)
    assert q.shape == (6, 128) and e.shape == (6, 4)
    for r in range(6):
        for b in range(4):
            blk = x[r, 32 * b:min(100, 32 * b + 32)]
            if blk.size == 0:
                assert e[r, b] == 127
                continue
            amax = float(np.max(np.abs(blk)))
            k = -127
            while k < 127 and not amax <= 448.0 * 2.0 ** k:
                k += 1
            assert e[r, b] == k + 127
            for i, v in enumerate(blk):
                y = float(v) * 2.0 ** -k
                assert abs(y) <= 448.0
                assert q[r, 32 * b + i] == brute_code_f64(y)
    assert np.all(q[:, 100:] == 0)
    assert e[0, 0] == 0 and np.all(q[0, :32] == 0)


def test_cols_is_rows_of_transpose_and_differs_from_transposed_rows():
    rng = np.random.default_rng(92)
    x = (rng.standard_normal((96, 64)) * np.exp(rng.uniform(-3, 3, (96, 64)))).astype(np.float32)
    qT, eT = oracle.mx_quant_cols(x)
    q2, e2 = oracle.mx_quant_rows(np.ascontiguousarray(x.T))
    assert np.array_equal(qT, q2) and np.array_equal(eT, e2)
    q, e = oracle.mx_quant_rows(x)
    assert not np.array_equal(qT[:, :96], q[:, :64].T)


def test_lossless_pow2_blocks():
    rng = np.random.default_rng(93)
    codes = rng.integers(0, 0x7E, size=(16, 256)) | (rng.integers(0, 2, (16, 256)) << 7)
    codes[:, ::32] = 0x7E
    k = rng.integers(-30, 30, size=(16, 8))
    x = (TABLE[codes] * np.repeat(np.ldexp(1.0, k), 32, axis=1)).astype(np.float32)
    q, e = oracle.mx_quant_rows(x)
    assert np.array_equal(e.astype(int) - 127, k)
    assert np.array_equal(oracle.deq_mx(q, e, 256), x.astype(np.float64))


def test_mx_gemm_exact_brute_force():
    rng = np.random.default_rng(94)
    K = 128
    A = (rng.standard_normal((2, K)) * np.exp(rng.uniform(-5, 5, (2, K)))).astype(np.float32)
    B = (rng.standard_normal((3, K)) * 0.02).astype(np.float32)
    aq, ae = oracle.mx_quant_rows(A)
    bq, be = oracle.mx_quant_rows(B)
    y = oracle.mx_gemm(aq, ae, bq, be, K)
    for i in range(2):
        for j in range(3):
            terms = [Fraction(float(TABLE[aq[i, k]])) * Fraction(2) ** (int(ae[i, k // 32]) - 127)
                     * Fraction(float(TABLE[bq[j, k]])) * Fraction(2) ** (int(be[j, k // 32]) - 127)
                     for k in range(K)]
            exact = sum(terms, Fraction(0))
            mag = sum(abs(float(t)) for t in terms)
            assert abs(float(Fraction(float(y[i, j])) - exact)) <= K * 2.0 ** -53 * mag * 1.01
