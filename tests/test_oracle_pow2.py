"""Pins for the oracle's power-of-two-scale quantizers (CPU only).

The SkyRL section on FP8 quantization with FP32 and power-of-two block
scales constrains each block scale to a power of two (an exponent-only
representation, up to a factor of two coarser).  The pages do not say how
the exponent is chosen; the reading used is the one the Miles MXFP8
paragraphs state for E8M0 scales: rounded up, so that the block maximum does
not clip.  Pins:

* closed form: S = 2^k with amax/448 <= S < 2 * amax/448 (an all-zero block
  takes 2^-127), checked with exact numpy arithmetic on every group;
* an independent encoder: with S a power of two the quotient x/S is exact,
  and the library's float8_e4m3fn conversion of it must give the same codes;
* agreement with the FP32-scale recipe wherever amax/448 is itself a power
  of two (the two rules then pick the same scale);
* the layout identities the FP32-scale quantizers obey (column-wise equals
  row-wise of the transpose, the transposed weight codes).
"""
import numpy as np
import torch

import oracle


def torch_codes(y: np.ndarray) -> np.ndarray:
    """E4M3 codes of exactly representable fp32 quotients, by torch."""
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def check_pow2_rule(amax: np.ndarray, S: np.ndarray):
    amax = amax.astype(np.float64)
    S64 = S.astype(np.float64)
    m, _ = np.frexp(S64)
    assert np.all(m == 0.5), "scale is not a power of two"
    zero = amax == 0
    assert np.all(S[zero] == np.float32(2.0 ** -127))
    nz = ~zero
    assert np.all(amax[nz] <= 448.0 * S64[nz]), "block maximum would clip"
    assert np.all(amax[nz] > 448.0 * S64[nz] / 2), "a smaller power of two would do"


def test_1x128_pow2_closed_form_and_library_codes():
    rng = np.random.default_rng(10)
    mags = np.exp(rng.uniform(-60, 60, (64, 1)))
    x = (rng.standard_normal((64, 300)) * mags).astype(np.float32)
    x[3] = 0.0
    x[4, :128] = -0.0
    q, s = oracle.quant_1x128(x, pow2=True)
    groups = [x[:, 0:128], x[:, 128:256], x[:, 256:300]]
    amax = np.stack([np.max(np.abs(g), axis=1) for g in groups], axis=1)
    check_pow2_rule(amax, s)
    for gi, g in enumerate(groups):
        y = g / s[:, gi:gi + 1]                                  # exact: S is a power of two
        want = torch_codes(y)
        assert np.array_equal(q[:, 128 * gi:128 * gi + g.shape[1]], want)
    assert np.all(q[:, 300:] == 0)
    assert np.all(q[4, :128] == 0x80)                           # signed zeros kept


def test_pow2_equals_fp32_rule_when_amax_is_448_times_power_of_two():
    rng = np.random.default_rng(11)
    k = rng.integers(-100, 100, 200)
    amax = (448.0 * np.ldexp(1.0, k)).astype(np.float32)
    x = (rng.uniform(-1, 1, (200, 128)) * amax[:, None]).astype(np.float32)
    x[:, 7] = amax
    q2, s2 = oracle.quant_1x128(x, pow2=True)
    q1, s1 = oracle.quant_1x128(x)
    assert np.array_equal(s1, s2)
    assert np.array_equal(q1, q2)


def test_pow2_scale_is_never_finer_than_fp32_scale():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((100, 256)) * np.exp(rng.uniform(-30, 30, (100, 1)))).astype(np.float32)
    _, s2 = oracle.quant_1x128(x, pow2=True)
    _, s1 = oracle.quant_1x128(x)
    assert np.all(s2 >= s1) and np.all(s2 < 2 * s1)


def test_128x128_pow2_closed_form_transpose_and_codes():
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((300, 260)) * 0.02).astype(np.float32)
    w[:128, 128:256] *= 1e20                                     # one hot tile
    q, s, qT = oracle.quant_128x128(w, pow2=True)
    amax = np.array([[np.max(np.abs(w[128 * i:128 * i + 128, 128 * j:128 * j + 128]))
                      for j in range(3)] for i in range(3)])
    check_pow2_rule(amax, s)
    for i in range(3):
        for j in range(3):
            t = w[128 * i:128 * i + 128, 128 * j:128 * j + 128]
            assert np.array_equal(q[128 * i:128 * i + t.shape[0], 128 * j:128 * j + t.shape[1]],
                                  torch_codes(t / s[i, j]))
    assert np.array_equal(qT[:, :300], q[:, :260].T)


def test_colwise_pow2_equals_rowwise_pow2_of_transpose_and_segments():
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((300, 40)) * 3.0).astype(np.float32)
    qT, sT = oracle.quant_colwise(x, pow2=True)
    q2, s2 = oracle.quant_1x128(np.ascontiguousarray(x.T), pow2=True)
    assert np.array_equal(qT, q2) and np.array_equal(sT, s2)
    offsets = np.array([0, 0, 130, 131, 300], dtype=np.int32)
    qT, sT = oracle.quant_colwise(x, offsets, pow2=True)
    P = oracle.padded_offsets(offsets)
    for e in range(4):
        a, b = offsets[e], offsets[e + 1]
        if b == a:
            continue
        qe, se = oracle.quant_1x128(np.ascontiguousarray(x[a:b].T), pow2=True)
        n = (b - a + 127) // 128
        assert np.array_equal(sT[:, P[e] // 128:P[e] // 128 + n], se)
        assert np.array_equal(qT[:, P[e]:P[e] + 128 * n], qe)


def test_e8m0_bytes_of_pow2_scales():
    s = np.array([2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0 ** 120], dtype=np.float32)
    assert list(oracle.e8m0_of_pow2(s)) == [0, 1, 126, 127, 247]
