"""Pins for the oracle's token-axis requantization from saved 1x128 FP8
data (CPU only).  The flow keeps only the FP8 activations and forms WGrad's
X^T from them (the Jet-RL pages describe it as the DeepSeek-V3 recipe).
Pins:

* the dequantization step against an independent one: torch's
  float8_e4m3fn decode of the codes times the scale in numpy float32, fed
  to the (separately pinned) token-axis quantizer;
* a lossless construction: when every 1x128 group holds E4M3 values times a
  power of two with its maximum at 448 times that power, dequantization
  returns the input exactly, so requantizing equals quantizing the input;
* grouped segments restart exactly as the token-axis quantizer's do.
"""
import numpy as np
import torch

import oracle


def np_dequant(q, s, cols):
    v = torch.from_numpy(np.ascontiguousarray(q[:, :cols])).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    sc = np.repeat(s, 128, axis=1)[:, :cols].astype(np.float32)
    return (v * sc).astype(np.float32)


def test_requant_equals_colwise_of_independent_dequant():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((300, 260)) * np.exp(rng.uniform(-10, 10, (300, 1)))).astype(np.float32)
    q, s = oracle.quant_1x128(x)
    qT, sT = oracle.requant_colwise(q, s, 260)
    wT, wsT = oracle.quant_colwise(np_dequant(q, s, 260))
    assert np.array_equal(qT, wT) and np.array_equal(sT.view(np.uint32), wsT.view(np.uint32))


def test_requant_lossless_groups_equal_direct_quantization():
    rng = np.random.default_rng(22)
    table = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    rows, cols = 256, 384
    codes = rng.choice(finite, (rows, cols))
    k = rng.integers(-20, 20, (rows, cols // 128))
    x = table[codes] * np.repeat(np.ldexp(1.0, k), 128, axis=1)
    for g in range(cols // 128):                                  # group maximum at 448 * 2^k
        x[np.arange(rows), 128 * g + rng.integers(0, 128, rows)] = 448.0 * np.ldexp(1.0, k[:, g])
    x = x.astype(np.float32)
    q, s = oracle.quant_1x128(x)
    assert np.array_equal(np_dequant(q, s, cols), x)              # lossless round trip
    qT, sT = oracle.requant_colwise(q, s, cols)
    wT, wsT = oracle.quant_colwise(x)
    assert np.array_equal(qT, wT) and np.array_equal(sT, wsT)


def test_requant_grouped_segments():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((300, 70)).astype(np.float32)
    q, s = oracle.quant_1x128(x)
    offsets = np.array([0, 0, 130, 131, 300], dtype=np.int32)
    qT, sT = oracle.requant_colwise(q, s, 70, offsets)
    wT, wsT = oracle.quant_colwise(np_dequant(q, s, 70), offsets)
    assert np.array_equal(qT, wT) and np.array_equal(sT.view(np.uint32), wsT.view(np.uint32))
