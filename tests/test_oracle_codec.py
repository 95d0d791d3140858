"""Pins for the oracle's E4M3 codec (CPU only).

The oracle's encoder is a bisection over its value table.  It is pinned here
against things other than itself:

* PyTorch's float8_e4m3fn dtype (an independent library implementation of
  the OCP E4M3 format that the Jet-RL notes cite for Delta_max = 448):
  its decode of all 256 codes, and its round-to-nearest-even cast over every
  fp32 value in [2^-11, 464) -- the cast produces NaN instead of saturating
  above that, so saturation is pinned by closed form instead;
* an independent bit-manipulation encoder written below;
* closed forms: everything below 2^-10 in magnitude encodes to a signed zero,
  everything at or above 448 saturates, the midpoint ties go to even codes.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def torch_decode_table() -> np.ndarray:
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bits_encoder(v: np.ndarray) -> np.ndarray:
    """Independent RNE-saturating E4M3 encoder working on the fp32 bits."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.int32)
    mag = u & np.int32(0x7FFFFFFF)
    af = mag.view(np.float32)
    # normal E4M3 range: keep 3 mantissa bits, round the 20 dropped bits
    base = (mag >> 20) - ((127 - 7) << 3)          # (e+7)<<3 | top 3 mantissa bits
    low = mag & np.int32(0xFFFFF)
    up = (low > 0x80000) | ((low == 0x80000) & ((base & 1) == 1))
    code = base + up
    # subnormal E4M3 range: value / 2^-9 rounded half-to-even
    sub = af < np.float32(2.0 ** -6)
    code[sub] = np.rint(af[sub] * np.float32(512.0)).astype(np.int32)
    code[af >= np.float32(448.0)] = 0x7E
    return (code | ((u >> 31) & 1) << 7).astype(np.uint8)


def test_page_constant_delta_max():
    g = json.load(open(GOLDEN))
    table = oracle.e4m3_decode_table()
    finite = table[~np.isnan(table)]
    assert finite.max() == g["e4m3_max"]["value"]
    assert oracle.e4m3_encode_f64(1e30) == 0x7E


def test_decode_table_matches_library():
    ours = oracle.e4m3_decode_table()
    ref = torch_decode_table()
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(ref))
    assert set(np.nonzero(nan_ours)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan_ours], ref[~nan_ours])
    # signed zeros
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_decode_spot_values():
    t = oracle.e4m3_decode_table()
    assert t[0x7E] == 448.0
    assert t[0x38] == 1.0
    assert t[0x08] == 2.0 ** -6
    assert t[0x01] == 2.0 ** -9
    assert t[0x07] == 7 * 2.0 ** -9
    assert t[0xFE] == -448.0
    # magnitudes strictly increase with the code over 0x00..0x7E
    assert np.all(np.diff(t[0:0x7F]) > 0)


def test_encode_roundtrip_all_finite_codes():
    t = oracle.e4m3_decode_table()
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode_f64(t[c]) == c, hex(c)


def test_encode_closed_form_points():
    enc = oracle.e4m3_encode_f64
    assert enc(448.0 * (1 + 2.0 ** -23)) == 0x7E
    assert enc(464.0) == 0x7E
    assert enc(1e30) == 0x7E
    assert enc(-1e30) == 0xFE
    assert enc(2.0 ** -10) == 0x00           # tie between 0 and 2^-9 -> even (0)
    assert enc(-2.0 ** -10) == 0x80
    assert enc(1.5 * 2.0 ** -9) == 0x02      # tie between codes 1 and 2 -> even
    assert enc(2.5 * 2.0 ** -9) == 0x02      # tie between codes 2 and 3 -> even
    assert enc(-0.0) == 0x80
    assert enc(0.0) == 0x00
    # midpoint between 1.0 (0x38) and 1.125 (0x39): even code 0x38
    assert enc(1.0625) == 0x38
    # midpoint between 1.125 (0x39) and 1.25 (0x3A): even code 0x3A
    assert enc(1.1875) == 0x3A
    # just above / below a midpoint
    assert enc(np.nextafter(1.0625, 2.0)) == 0x39
    assert enc(np.nextafter(1.1875, 0.0)) == 0x39


def test_every_midpoint_goes_to_even_code():
    t = oracle.e4m3_decode_table()
    for c in range(0, 0x7E):
        mid = 0.5 * (t[c] + t[c + 1])
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode_f64(mid) == want
        assert oracle.e4m3_encode_f64(-mid) == want | 0x80


def _sweep(lo_bits: int, hi_bits: int, chunk: int = 1 << 22):
    for start in range(lo_bits, hi_bits, chunk):
        stop = min(hi_bits, start + chunk)
        yield np.arange(start, stop, dtype=np.uint32).view(np.float32)


def test_encode_exhaustive_core_range_vs_bits_encoder():
    """Every fp32 value with 2^-11 <= |v| < 2^9, both signs."""
    lo, hi = 0x3A000000, 0x44000000
    for v in _sweep(lo, hi):
        ours = oracle.e4m3_encode(v)
        assert np.array_equal(ours, bits_encoder(v))
        neg = -v
        assert np.array_equal(oracle.e4m3_encode(neg), bits_encoder(neg))


def test_encode_exhaustive_core_range_vs_library():
    """torch's float8_e4m3fn cast is RNE; it agrees wherever it does not
    overflow (|v| < 464)."""
    lo, hi = 0x3A000000, int(np.float32(464.0).view(np.uint32))
    for v in _sweep(lo, hi):
        ours = oracle.e4m3_encode(v)
        ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(ours, ref)


def test_encode_outside_core_range_closed_form():
    """Below 2^-10 the nearest E4M3 value is a signed zero (ties included);
    at or above 448 the encoder saturates.  Checked on a dense stride over
    both regions (every 97th fp32 pattern) plus their edges."""
    small = np.arange(0, 0x3A800001, 97, dtype=np.uint32)
    small = np.concatenate([small, np.array([0x3A800000, 0x3A7FFFFF, 1, 0x007FFFFF, 0x00800000],
                                            dtype=np.uint32)]).view(np.float32)
    assert np.all(oracle.e4m3_encode(small) == 0x00)
    assert np.all(oracle.e4m3_encode(-small) == 0x80)
    big = np.arange(int(np.float32(448.0).view(np.uint32)), 0x7F800000, 97, dtype=np.uint32)
    big = np.concatenate([big, np.array([0x7F7FFFFF], dtype=np.uint32)]).view(np.float32)
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)
    # the first fp32 value above 2^-10 rounds up to the smallest subnormal
    assert oracle.e4m3_encode_f64(np.nextafter(2.0 ** -10, 1.0)) == 0x01
