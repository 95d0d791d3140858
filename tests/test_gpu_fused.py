"""GPU parity of the fused producers of the 1x128 activation quantizer
against the oracle, bit for bit: codes, scales, the bf16 activation and
RMSNorm's per-row r.

* SiLU(gate) * up: every finite bf16 gate value (with up = 1 the activation
  is silu(g) itself, so the whole SiLU table is checked), ragged shapes with
  gate and up as views of one gate+up matrix, and the training shape
  (8192 x 12288) on sampled rows;
* RMSNorm: bf16 and fp32 inputs and weights, two epsilons, ragged widths
  for every register-resident pass count (1, 2, 4 and 8 passes of 1024
  columns), a width past that limit (re-read path), rows whose
  magnitudes span 2^30, and the decode/training hidden width on sampled rows;
* both equal the unfused path: the 1x128 quantizer run on the fused kernel's
  own bf16 output gives the same codes and scales;
* the bf16 rounding both producers use (the packed hardware conversion) on
  every non-NaN fp32 bit pattern.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_02_amd as fb
import oracle
from block_scaled_fp8_02_amd import workloads as wl
from gpu_util import assert_bytes_equal, assert_scales_equal, banner, dev, dev_strided, host

pytestmark = pytest.mark.gpu


def bits_of(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> host uint16 bits."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).to("cuda")


def gate_up_views(gate: np.ndarray, up: np.ndarray):
    """gate and up as the two halves of one [rows, 2*cols(+pad)] bf16 matrix."""
    rows, cols = gate.shape
    pad = (-cols) % 8
    H = np.zeros((rows, 2 * (cols + pad)), np.uint16)
    H[:, :cols] = gate
    H[:, cols + pad:2 * cols + pad] = up
    Hd = bf16_dev(H)
    return Hd[:, :cols], Hd[:, cols + pad:2 * cols + pad]


def test_bf16_rounding_every_fp32_pattern():
    """The producers round their activations to bf16 with the packed
    conversion; on every finite and infinite fp32 value it must give the
    oracle's nearest-even bits."""
    banner("bf16 rounding over all 2^32 fp32 patterns")
    step = 1 << 28
    for lo in range(-(1 << 31), 1 << 31, step):
        banner(f"bf16 chunk {lo:#x}")
        x = torch.arange(lo, lo + step, dtype=torch.int32, device="cuda").view(torch.float32)
        got = fb.fp8b_bf16_round(x).cpu().numpy().view(np.uint16)
        xs = np.arange(lo, lo + step, dtype=np.int64).astype(np.int32).view(np.float32)
        keep = ~np.isnan(xs)
        want = oracle.bf16_rne(xs[keep])
        assert_bytes_equal(got[keep], want, f"bf16 rounding chunk at {lo:#x}")
        del x


def check_silu(gate: np.ndarray, up: np.ndarray, what: str):
    gd, ud = gate_up_views(gate, up)
    q, s, a = fb.fp8_silu_mul_quantize_1x128(gd, ud, a=True)
    wq, ws, wa = oracle.silu_mul_quant_1x128(gate, up)
    assert_bytes_equal(bits_of(a), wa, f"{what} activation")
    assert_bytes_equal(host(q), wq, f"{what} codes")
    assert_scales_equal(host(s), ws, f"{what} scales")
    q2, s2 = fb.fp8_quantize_act_1x128(a)
    assert torch.equal(q, q2) and torch.equal(s, s2), f"{what}: fused != unfused"


def test_silu_every_finite_bf16_gate():
    banner("silu: all 65280 finite bf16 gate values, up = 1")
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = allb[(allb & 0x7F80) != 0x7F80]
    gate = finite.reshape(510, 128)
    up = np.full(gate.shape, 0x3F80, np.uint16)
    check_silu(gate, up, "silu table")
    # the same gates against varied up values, |up| < 1 so that no product
    # leaves the finite range (the activation must be finite)
    rng = np.random.default_rng(50)
    up2 = oracle.bf16_rne((rng.uniform(-1, 1, gate.shape) * np.exp(rng.uniform(-30, 0, gate.shape)))
                          .astype(np.float32))
    check_silu(gate, up2, "silu table x random up")


@pytest.mark.parametrize("shape", [(1, 1), (3, 300), (129, 257), (64, 1000), (17, 2048)])
def test_silu_mul_ragged(shape):
    banner(f"silu*up {shape}")
    rng = np.random.default_rng(sum(shape) + 51)
    g = oracle.bf16_rne((rng.standard_normal(shape) * 3).astype(np.float32))
    u = oracle.bf16_rne((rng.standard_normal(shape) * np.exp(rng.uniform(-10, 10, (shape[0], 1))))
                        .astype(np.float32))
    check_silu(g, u, f"silu*up {shape}")


def test_silu_mul_training_shape_sampled_rows():
    """Down-projection input of the training layer: gate, up [8192 x 12288]
    (one gate+up matrix [8192 x 24576]); 32 sampled rows against the oracle."""
    N, I = 8192, 12288
    banner(f"silu*up training shape {N}x{I}")
    rng = wl.rng_for(7)
    H = wl.normal_bf16(rng, (N, 2 * I), 1.0)
    Hd = bf16_dev(H)
    q, s, a = fb.fp8_silu_mul_quantize_1x128(Hd[:, :I], Hd[:, I:], a=True)
    rows = np.sort(np.random.default_rng(52).choice(N, 32, replace=False))
    wq, ws, wa = oracle.silu_mul_quant_1x128(H[rows, :I], H[rows, I:])
    assert_bytes_equal(bits_of(a)[rows], wa, "training silu activation (sampled rows)")
    assert_bytes_equal(host(q)[rows], wq, "training silu codes (sampled rows)")
    assert_scales_equal(host(s)[rows], ws, "training silu scales (sampled rows)")


def check_rmsnorm(x: np.ndarray, w: np.ndarray, eps: float, what: str, strided: bool = True):
    xd = dev_strided(x) if strided else dev(x)
    wd = dev(w)
    q, s, r, y = fb.fp8_rmsnorm_quantize_1x128(xd, wd, eps, rstd=True, y=True)
    wq, ws, wr, wy = oracle.rmsnorm_quant_1x128(x, w, eps)
    assert_scales_equal(host(r), wr, f"{what} rstd")
    assert_bytes_equal(bits_of(y), wy, f"{what} y")
    assert_bytes_equal(host(q), wq, f"{what} codes")
    assert_scales_equal(host(s), ws, f"{what} scales")
    q2, s2 = fb.fp8_quantize_act_1x128(y)
    assert torch.equal(q, q2) and torch.equal(s, s2), f"{what}: fused != unfused"


@pytest.mark.parametrize("shape", [(1, 1), (3, 300), (129, 257), (7, 1500), (64, 4096), (9, 6000), (5, 20000)])
@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_rmsnorm_ragged(shape, kind):
    banner(f"rmsnorm {kind} {shape}")
    rng = np.random.default_rng(sum(shape) + (53 if kind == "bf16" else 54))
    x = (rng.standard_normal(shape) * np.exp(rng.uniform(-8, 8, (shape[0], 1)))).astype(np.float32)
    w = (1 + 0.2 * rng.standard_normal(shape[1])).astype(np.float32)
    if kind == "bf16":
        x, w = oracle.bf16_rne(x), oracle.bf16_rne(w)
    for eps in (1e-6, 0.5):
        check_rmsnorm(x, w, eps, f"rmsnorm {kind} {shape} eps {eps}")


def test_rmsnorm_mixed_input_and_weight_types_and_wide_rows():
    banner("rmsnorm mixed dtypes, rows spanning 2^30")
    rng = np.random.default_rng(55)
    sign = np.where(rng.random((40, 1024)) < 0.5, -1.0, 1.0)
    x = (sign * np.exp2(rng.uniform(-15, 15, (40, 1024)))).astype(np.float32)
    w = (1 + 0.2 * rng.standard_normal(1024)).astype(np.float32)
    x[3] = 0.0                                                       # all-zero row: r = fl32(1/sqrt(eps))
    x[4, :] = np.float32(2.0 ** -60)
    check_rmsnorm(oracle.bf16_rne(x), w, 1e-6, "bf16 x, fp32 w")
    check_rmsnorm(x, oracle.bf16_rne(w), 1e-6, "fp32 x, bf16 w")


def test_rmsnorm_hidden_width_sampled_rows():
    """RMSNorm before the gate/up and QKV projections at the training
    shape: x bf16 [8192 x 4096] (the hidden width), w bf16 around 1."""
    N, H = 8192, 4096
    banner(f"rmsnorm training shape {N}x{H}")
    rng = wl.rng_for(8)
    x = wl.normal_bf16(rng, (N, H), 1.0)
    w = wl.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    q, s, r, y = fb.fp8_rmsnorm_quantize_1x128(dev(x), dev(w), 1e-6, rstd=True, y=True)
    rows = np.sort(np.random.default_rng(56).choice(N, 64, replace=False))
    wq, ws, wr, wy = oracle.rmsnorm_quant_1x128(x[rows], w, 1e-6)
    assert_scales_equal(host(r)[rows], wr, "training rstd (sampled rows)")
    assert_bytes_equal(bits_of(y)[rows], wy, "training y (sampled rows)")
    assert_bytes_equal(host(q)[rows], wq, "training codes (sampled rows)")
    assert_scales_equal(host(s)[rows], ws, "training scales (sampled rows)")
