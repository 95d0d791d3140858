"""CPU oracle for the fused producers of the 1x128 activation quantizer:
RMSNorm + quantize and SiLU(gate) * up + quantize.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain numpy and
Python, no code shared with the HIP library.

The Jet-RL notes (section 3.4 and the per-block walk-through of the
attention and MLP blocks) fuse the 1x128 activation quantization into the
operator that produces the activation, so that the bf16 activation is not
written to memory and read back.  The pages do not define the operators'
arithmetic; the readings taken here:

* RMSNorm, for one row x of C values with weight w and epsilon eps:
  ss = sum of x_j^2, exact, rounded once to binary64; r = fl32(1 / sqrt(ss / C
  + eps)) with the division, addition, square root and reciprocal each a
  binary64 operation; y_j = bf16(fl32(fl32(x_j * r) * w_j)).  The output
  is the bf16 activation the unfused graph would hand to the quantizer, so
  the fused result equals "RMSNorm to bf16, then the 1x128 quantizer".
* SiLU and the elementwise product, "computed in BF16" in the notes'
  MLP walk-through: s = bf16(silu(g)) rounded once from the exact value
  g / (1 + e^-g), then a = bf16(fl32(s * u)), then the 1x128 quantizer.

bf16(.) is IEEE round-to-nearest-even into bfloat16 (8 significant bits,
binary32's exponent range, subnormals kept, overflow to infinity).
"""
from __future__ import annotations

import math

import numpy as np


# ------------------------------------------------------------ bfloat16
def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 bits (uint16) of finite float32 values: the upper
    16 bits of the float32 pattern after adding half of the dropped part,
    ties going to the even result."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    return ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_rne_from_f64(d: np.ndarray, rsign: np.ndarray | None = None) -> np.ndarray:
    """Nearest-even bf16 bits of t = d + delta, rounded once, where d is a
    binary64 value and delta a residual far below d's binary32 spacing whose
    sign is rsign (-1, 0 or +1; None: all 0, t = d).  t is first rounded to
    binary32 with round-to-odd (of the two binary32 values enclosing t, the
    one with an odd last bit; t itself when representable), then to bf16
    with nearest-even.  binary32 carries at least two bits more than bf16
    over the whole range, so the two steps equal one direct rounding of t
    (Boldo and Melquiond, "Emulation of FMA and correctly rounded sums:
    proved algorithms using rounding to odd", IEEE Trans. Computers 57(4),
    2008).  Values beyond the binary32 range are not valid inputs."""
    d = np.asarray(d, dtype=np.float64)
    rs = np.zeros(d.shape, dtype=np.int64) if rsign is None else np.asarray(rsign, dtype=np.int64)
    f = d.astype(np.float32)                                   # nearest binary32 to d
    back = f.astype(np.float64)
    mag = np.abs(f).view(np.uint32).astype(np.int64)           # |f| as an ordered integer
    neg = np.signbit(d)
    # where t lies relative to |f|, in magnitude: +1 above, -1 below, 0 on it
    side = np.where(np.abs(d) > np.abs(back), 1, np.where(np.abs(d) < np.abs(back), -1, 0))
    side = np.where(side == 0, np.where(neg, -rs, rs), side)
    side = np.where((d == 0) & (rs != 0), 1, side)             # t = +-delta: above zero in magnitude
    neg = np.where((d == 0) & (rs != 0), rs < 0, neg)
    odd = (mag & 1) == 1
    ro = np.where((side == 0) | odd, mag, mag + side)          # the odd one of the enclosing pair
    bits = (ro.astype(np.uint32) | (neg.astype(np.uint32) << 31)).view(np.float32)
    return bf16_rne(bits)


# -------------------------------------------------------------- RMSNorm
def rmsnorm_sumsq(x: np.ndarray) -> np.ndarray:
    """Per-row exact sum of squares rounded once to binary64."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    return np.array([math.fsum((row * row).tolist()) for row in x64], dtype=np.float64)


def rmsnorm_rstd(x: np.ndarray, eps: float) -> np.ndarray:
    """Per-row r = fl32(1 / sqrt(ss / C + eps)) with ss the exact sum of
    squares rounded once to binary64 (math.fsum of the squares, each exact in
    binary64 for bf16 and fp32 inputs)."""
    x = np.asarray(x, dtype=np.float32)
    rows, C = x.shape
    r = np.empty(rows, dtype=np.float32)
    sums = rmsnorm_sumsq(x)
    for i in range(rows):
        t = float(sums[i]) / float(C)
        t = t + float(np.float32(eps))
        t = math.sqrt(t)
        r[i] = np.float32(1.0 / t)
    return r


def rmsnorm_bf16(x: np.ndarray, w: np.ndarray, eps: float):
    """RMSNorm rows of x (float32 values; bf16 inputs widened exactly) with
    weight w [C].  Returns (y bf16 bits [rows, C], r float32 [rows])."""
    x = np.asarray(x, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32)
    r = rmsnorm_rstd(x, eps)
    xr = (x * r[:, None]).astype(np.float32)                 # binary32 products
    y = (xr * w[None, :]).astype(np.float32)
    return bf16_rne(y), r


# ----------------------------------------------------------------- SiLU
_SILU_TABLE = None


def silu_table() -> np.ndarray:
    """bf16 bits of silu(g) for every bf16 bit pattern g (NaN and infinity
    patterns map to themselves; they are not valid inputs).  silu(g) =
    g / (1 + e^-g) in binary64, written for negative g as g e^g / (1 + e^g)
    so that nothing overflows, then rounded once to bf16."""
    global _SILU_TABLE
    if _SILU_TABLE is not None:
        return _SILU_TABLE
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        g = bf16_to_f32(bits).astype(np.float64)
    finite = np.isfinite(g)
    gs = np.where(finite, g, 0.0)
    with np.errstate(over="ignore", under="ignore"):
        pos = gs / (1.0 + np.exp(-np.abs(gs)))               # used where g >= 0
        e = np.exp(-np.abs(gs))
        neg = gs * e / (1.0 + e)                             # used where g < 0
    v = np.where(gs >= 0, pos, neg)
    # |g| < 2^-100: silu(g) = g/2 + g^2/4 - ..., with g/2 exact and the rest a
    # positive residual far below binary32 spacing (binary64 would drop it,
    # and for subnormal g that decides ties: g/2 is then a bf16 midpoint)
    tiny = (np.abs(gs) < 2.0 ** -100) & (gs != 0)
    v = np.where(tiny, gs / 2.0, v)
    v = np.where(gs == 0, gs, v)                             # silu(+-0) = +-0
    out = bf16_rne_from_f64(v, np.where(tiny, 1, 0))
    out = np.where(finite, out, bits)
    _SILU_TABLE = out.astype(np.uint16)
    return _SILU_TABLE


def silu_mul_bf16(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """a = bf16(fl32(bf16(silu(g)) * u)) for bf16 bit arrays gate and up."""
    s = silu_table()[np.asarray(gate, dtype=np.uint16)]
    prod = (bf16_to_f32(s) * bf16_to_f32(up)).astype(np.float32)
    return bf16_rne(prod)
