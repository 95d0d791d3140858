"""Pins for the oracle's bf16 dequantization of FP8 operands (CPU only),
the operands of the dequantized-backward mode the Miles MXFP8/NVFP4 blog
describes: bf16(fl32(E4M3(q) * s)).  Checked against an independent path:
torch's float8_e4m3fn decode, a float32 multiply by the scale, and torch's
float32 -> bfloat16 conversion; plus the exact case (power-of-two scales
give a bf16-exact product) and the scale layouts (which scale each element
uses)."""
import numpy as np
import torch

import oracle


def torch_deq(q: np.ndarray, scale_per_elem: np.ndarray) -> np.ndarray:
    v = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float32)
    p = v * torch.from_numpy(np.ascontiguousarray(scale_per_elem, dtype=np.float32))
    return p.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E                         # no NaN codes
    return c


def test_rows_1x128_against_torch():
    rng = np.random.default_rng(60)
    q = codes(rng, (50, 384))
    s = (rng.uniform(0.5, 2, (50, 3)) * np.exp(rng.uniform(-60, 60, (50, 3)))).astype(np.float32)
    got = oracle.dequant_bf16_rows(q, s, 300)
    want = torch_deq(q[:, :300], np.repeat(s, 128, axis=1)[:, :300])
    assert np.array_equal(got, want)


def test_128x128_against_torch_and_layout():
    rng = np.random.default_rng(61)
    q = codes(rng, (300, 384))
    s = (rng.uniform(0.5, 2, (3, 3)) * 1e-3).astype(np.float32)
    got = oracle.dequant_bf16_128x128(q, s, 300, 260)
    per = np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)[:300, :260]
    assert np.array_equal(got, torch_deq(q[:, :260], per))
    # block (1, 2) alone: changing its scale changes exactly rows 128..255, cols 256..259
    s2 = s.copy()
    s2[1, 2] *= 3
    diff = oracle.dequant_bf16_128x128(q, s2, 300, 260) != got
    rows, cols = np.nonzero(diff)
    assert rows.min() >= 128 and rows.max() < 256 and cols.min() >= 256


def test_mx_against_torch_and_power_of_two_exactness():
    rng = np.random.default_rng(62)
    q = codes(rng, (40, 256))
    e = rng.integers(80, 170, (40, 8)).astype(np.uint8)
    got = oracle.dequant_bf16_mx(q, e, 256)
    per = np.repeat(np.ldexp(1.0, e.astype(np.int64) - 127), 32, axis=1).astype(np.float32)
    assert np.array_equal(got, torch_deq(q, per))
    # an E4M3 value times a power of two is exact in bf16 (4 <= 8 significant bits)
    back = oracle.bf16_to_f32(got).astype(np.float64)
    assert np.array_equal(back, oracle.deq_mx(q, e, 256))
