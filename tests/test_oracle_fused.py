"""Pins for the oracle's fused producers (CPU only): RMSNorm + 1x128 and
SiLU(gate) * up + 1x128 (oracle/fused.py states the readings).

* bf16 rounding: against torch's float32 -> bfloat16 conversion, and the
  one-step rounding from binary64 against exact rational rounding;
* SiLU: every finite bf16 input against silu evaluated to 60 decimal digits
  (Python's decimal module) and rounded by exact comparison with the bf16
  midpoints around it, so the table is right for all 65280 inputs;
* the product step against the exact rational product rounded to bf16;
* RMSNorm: the exact sum of squares against rational arithmetic on rows
  where naive summation is not exact, r and y against torch's rms_norm in
  binary64, the closed form for constant rows, and invariance of y under
  scaling x by powers of two when eps is 0.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def bf16_value(bits: int) -> Fraction:
    f = float(oracle.bf16_to_f32(np.array([bits], dtype=np.uint16))[0])
    return Fraction(f)


def order_key(bits: int) -> int:
    """Monotone integer for bf16 bit patterns (both zeros map to 0)."""
    return bits if bits < 0x8000 else -(bits & 0x7FFF)


def from_key(k: int) -> int:
    return k if k >= 0 else (0x8000 | (-k))


def nearest_bf16_ok(exact: Fraction, bits: int) -> bool:
    """bits is the nearest-even bf16 to `exact` (finite, both neighbors
    finite): exact lies within the midpoints to the neighbors, and on a tie
    the even pattern won."""
    k = order_key(bits)
    v = bf16_value(bits)
    lo, hi = bf16_value(from_key(k - 1)), bf16_value(from_key(k + 1))
    m_lo, m_hi = (v + lo) / 2, (v + hi) / 2
    if m_lo < exact < m_hi:
        return True
    if exact == m_lo or exact == m_hi:
        return (bits & 1) == 0
    return False


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(40)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-80, 80, 200000))).astype(np.float32)
    ties = (rng.integers(0, 2 ** 16, 5000).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)], np.float32([0.0, -0.0, 1e-45, -1e-45, 3.3e38])])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_rne(x), want)


def test_bf16_rne_from_f64_is_one_rounding():
    rng = np.random.default_rng(41)
    d = rng.standard_normal(3000) * np.exp(rng.uniform(-90, 85, 3000))
    # doubles just beside and exactly on bf16 midpoints (normal and subnormal)
    mids = []
    for b in rng.integers(1, 0x7F00, 300):
        m = (bf16_value(int(b)) + bf16_value(int(b) + 1)) / 2
        mids += [float(m), math.nextafter(float(m), 0.0), math.nextafter(float(m), math.inf)]
    d = np.concatenate([d, np.array(mids), -np.array(mids), [2.0 ** -134, 2.0 ** -140, 0.0]])
    got = oracle.bf16_rne_from_f64(d)
    for v, b in zip(d, got):
        assert nearest_bf16_ok(Fraction(float(v)), int(b)), (v, hex(int(b)))
    # with a residual: t = d + delta, delta of the given sign and far below
    # binary32 spacing (exact midpoints, and binary32 values, pushed either way)
    base = np.array(mids + [float(bf16_value(int(b))) for b in rng.integers(1, 0x7F00, 200)])
    base = np.concatenate([base, -base])
    for sgn in (-1, 1):
        got = oracle.bf16_rne_from_f64(base, np.full(base.size, sgn))
        for v, b in zip(base, got):
            exact = Fraction(float(v)) + sgn * abs(Fraction(float(v))) * Fraction(1, 2 ** 80)
            assert nearest_bf16_ok(exact, int(b)), (v, sgn, hex(int(b)))


def test_silu_table_every_bf16_input_against_decimal():
    getcontext().prec = 60
    table = oracle.silu_table()
    checked = 0
    for bits in range(65536):
        if (bits & 0x7F80) == 0x7F80:                     # inf / NaN patterns
            continue
        g = float(bf16_value(bits))
        got = int(table[bits])
        checked += 1
        if g == 0.0:
            assert got == bits                            # silu(+-0) = +-0
            continue
        if g > 200:
            assert got == bits                            # g (1 - e^-g) rounds to g
            continue
        if g < -200:
            assert got == 0x8000                          # |g e^g| far below half the bf16 minimum
            continue
        G = Decimal(g)
        v = G / (1 + (-G).exp())
        exact = Fraction(v)
        assert nearest_bf16_ok(exact, got), (hex(bits), g, hex(got))
        # the 60-digit value is far from any midpoint: the decision is certain
        k = order_key(got)
        for nb in (from_key(k - 1), from_key(k + 1)):
            m = (bf16_value(got) + bf16_value(nb)) / 2
            assert abs(exact - m) > abs(exact) * Fraction(1, 10 ** 50)
    assert checked == 65536 - 256                          # every finite pattern


def test_silu_mul_product_rounds_the_exact_product():
    rng = np.random.default_rng(42)
    g = oracle.bf16_rne((rng.standard_normal(4000) * 3).astype(np.float32))
    u = oracle.bf16_rne((rng.standard_normal(4000) * np.exp(rng.uniform(-20, 20, 4000))).astype(np.float32))
    a = oracle.silu_mul_bf16(g, u)
    s = oracle.silu_table()[g]
    for si, ui, ai in zip(s, u, a):
        exact = bf16_value(int(si)) * bf16_value(int(ui))
        assert nearest_bf16_ok(exact, int(ai)), (hex(int(si)), hex(int(ui)), hex(int(ai)))


def test_rmsnorm_sum_of_squares_is_exact_then_rounded():
    rng = np.random.default_rng(43)
    rows = []
    for _ in range(20):
        r = (rng.standard_normal(300) * np.exp(rng.uniform(-40, 40, 300))).astype(np.float32)
        rows.append(r)
    r = np.zeros(300, np.float32)
    r[0], r[1:4] = 1.0, np.float32(2.0 ** -26.5)             # 1 + 3 * 2^-53: naive order gives 1
    rows.append(r)
    x = np.stack(rows)
    got = oracle.rmsnorm_sumsq(x)
    for row, g in zip(x, got):
        exact = sum(Fraction(float(v)) ** 2 for v in row)
        assert g == float(exact)                          # float(Fraction) rounds to nearest-even


@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_rmsnorm_against_torch_float64(eps):
    rng = np.random.default_rng(44)
    x = oracle.bf16_to_f32(oracle.bf16_rne(rng.standard_normal((16, 1000)).astype(np.float32)))
    w = oracle.bf16_to_f32(oracle.bf16_rne((1 + 0.1 * rng.standard_normal(1000)).astype(np.float32)))
    y, r = oracle.rmsnorm_bf16(x, w, eps)
    xt = torch.from_numpy(x.astype(np.float64))
    ref = torch.nn.functional.rms_norm(xt, (1000,), torch.from_numpy(w.astype(np.float64)), eps=float(np.float32(eps)))
    rr = torch.rsqrt((xt * xt).mean(dim=1) + float(np.float32(eps))).numpy()
    assert np.max(np.abs(r / rr - 1)) < 2.0 ** -23
    yv = oracle.bf16_to_f32(y).astype(np.float64)
    assert np.all(np.abs(yv - ref.numpy()) <= np.abs(ref.numpy()) * 2.0 ** -8 + 1e-30)


def test_rmsnorm_constant_rows_closed_form():
    c = np.float32([0.25, -8.0, 2.0 ** -60, -(2.0 ** 70)])
    x = np.repeat(c[:, None], 384, axis=1)
    y, r = oracle.rmsnorm_bf16(x, np.ones(384, np.float32), 0.0)
    assert np.array_equal(r, (1.0 / np.abs(c)).astype(np.float32))
    want = np.where(c > 0, 0x3F80, 0xBF80).astype(np.uint16)
    assert np.all(y == want[:, None])
    q, s, _, _ = oracle.rmsnorm_quant_1x128(x, np.ones(384, np.float32), 0.0)
    assert np.all(q[:, :384] == np.where(c > 0, 0x7E, 0xFE)[:, None])


def test_rmsnorm_power_of_two_scaling_invariance():
    rng = np.random.default_rng(45)
    x = oracle.bf16_to_f32(oracle.bf16_rne(rng.standard_normal((8, 500)).astype(np.float32)))
    w = (1 + 0.1 * rng.standard_normal(500)).astype(np.float32)
    y0, r0 = oracle.rmsnorm_bf16(x, w, 0.0)
    for k in (-30, -3, 5, 40):
        y1, r1 = oracle.rmsnorm_bf16((x * np.float32(2.0 ** k)).astype(np.float32), w, 0.0)
        assert np.array_equal(y0, y1)
        assert np.array_equal(r1, (r0 * np.float32(2.0 ** -k)).astype(np.float32))
