"""CPU oracle for the block-scaled FP8 linear-layer path (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The HIP library never imports,
links or calls anything here, and nothing here imports the HIP library.

Every function wraps ``fp8_oracle.c`` (plain C, fp32 IEEE quantization, fp64
GEMMs).  bf16 inputs arrive as their raw uint16 bits and are widened to fp32
here by a 16-bit left shift, which is exact.  Output layouts follow the C
file's comments: FP8 codes padded with 0x00 to a multiple of 128 along the
contraction axis, fp32 scales one per group.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(os.path.join(_HERE, "fp8_oracle.c"))
    ):
        from . import build as _build  # noqa: WPS433 (build on first use)

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.ora_e4m3_decode.restype = ctypes.c_double
    lib.ora_e4m3_decode.argtypes = [ctypes.c_int]
    lib.ora_e4m3_encode.restype = ctypes.c_uint8
    lib.ora_e4m3_encode.argtypes = [ctypes.c_float]
    lib.ora_e4m3_encode_f64.restype = ctypes.c_uint8
    lib.ora_e4m3_encode_f64.argtypes = [ctypes.c_double]
    lib.ora_e4m3_encode_array.argtypes = [_p, _i64, _p]
    lib.ora_quant_1x128.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _i64]
    lib.ora_quant_128x128.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64]
    lib.ora_quant_colwise.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64]
    lib.ora_quant_1x128_p2.argtypes = lib.ora_quant_1x128.argtypes
    lib.ora_requant_colwise.argtypes = [_p, _i64, _p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64]
    lib.ora_quant_128x128_p2.argtypes = lib.ora_quant_128x128.argtypes
    lib.ora_quant_colwise_p2.argtypes = lib.ora_quant_colwise.argtypes
    lib.ora_mx_exponent.restype = ctypes.c_int
    lib.ora_mx_exponent.argtypes = [ctypes.c_float]
    lib.ora_mx_quant_rows.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _i64]
    lib.ora_mx_quant_cols.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _i64]
    lib.ora_deq_rowgroups.argtypes = [_p, _i64, _p, _i64, _i64, _i64, _i64, _p, _i64]
    lib.ora_deq_128x128.argtypes = [_p, _i64, _p, _i64, _i64, _i64, _p, _i64]
    lib.ora_deq_mx.argtypes = [_p, _i64, _p, _i64, _i64, _i64, _p, _i64]
    lib.ora_matmul_f64.argtypes = [_p, _i64, _p, _i64, _i64, _i64, _i64, _p, _i64]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _rup(n: int, m: int) -> int:
    return (n + m - 1) // m * m


def _cdiv(n: int, m: int) -> int:
    return (n + m - 1) // m


def as_f32(x: np.ndarray) -> np.ndarray:
    """fp32 view of an input: float32 passes through, uint16 (bf16 bits)
    widens exactly by a 16-bit shift."""
    if x.dtype == np.float32:
        return np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    raise TypeError(f"oracle input must be float32 or bf16 bits (uint16), got {x.dtype}")


# ---------------------------------------------------------------- codec
def e4m3_decode_table() -> np.ndarray:
    lib = _load()
    return np.array([lib.ora_e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib.ora_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_encode_f64(v: float) -> int:
    return int(_load().ora_e4m3_encode_f64(float(v)))


# ---------------------------------------------------------- quantizers
def quant_1x128(x: np.ndarray, pow2: bool = False):
    """1x128 groups along the last axis.  Returns (q [rows, rup(cols,128)] u8,
    s [rows, ceil(cols/128)] f32); pow2 selects power-of-two scales."""
    lib = _load()
    x = as_f32(x)
    rows, cols = x.shape
    q = np.full((rows, _rup(cols, 128)), 0xAA, dtype=np.uint8)
    s = np.empty((rows, _cdiv(cols, 128)), dtype=np.float32)
    fn = lib.ora_quant_1x128_p2 if pow2 else lib.ora_quant_1x128
    fn(_ptr(x), rows, cols, cols, _ptr(q), q.shape[1], _ptr(s), s.shape[1])
    return q, s


def quant_128x128(w: np.ndarray, with_transpose: bool = True, pow2: bool = False):
    """128x128 blocks of W [D, C].  Returns (q [D, rup(C)], s [ceil(D/128),
    ceil(C/128)], qT [C, rup(D)] or None)."""
    lib = _load()
    w = as_f32(w)
    D, C = w.shape
    q = np.full((D, _rup(C, 128)), 0xAA, dtype=np.uint8)
    s = np.empty((_cdiv(D, 128), _cdiv(C, 128)), dtype=np.float32)
    qT = np.full((C, _rup(D, 128)), 0xAA, dtype=np.uint8) if with_transpose else None
    fn = lib.ora_quant_128x128_p2 if pow2 else lib.ora_quant_128x128
    fn(_ptr(w), D, C, C, _ptr(q), q.shape[1], _ptr(s), s.shape[1],
       _ptr(qT) if qT is not None else None, qT.shape[1] if qT is not None else 0)
    return q, s, qT


def padded_offsets(offsets: np.ndarray) -> np.ndarray:
    """Start of each segment in the transposed layout: segment e starts at
    sum_{e'<e} round_up(n_e', 128)."""
    n = np.diff(np.asarray(offsets, dtype=np.int64))
    return np.concatenate([[0], np.cumsum((n + 127) // 128 * 128)]).astype(np.int64)


def quant_colwise(x: np.ndarray, offsets: np.ndarray | None = None, pow2: bool = False):
    """1x128 groups along the token (row) axis, written transposed.  Returns
    (qT [cols, P] u8, sT [cols, P/128] f32) with P the padded token count;
    pow2 selects power-of-two scales."""
    lib = _load()
    x = as_f32(x)
    rows, cols = x.shape
    if offsets is None:
        P = _rup(rows, 128)
        offs_p, E = None, 0
    else:
        offsets = np.ascontiguousarray(offsets, dtype=np.int32)
        E = offsets.size - 1
        P = int(padded_offsets(offsets)[-1])
        offs_p = _ptr(offsets)
    qT = np.full((cols, max(P, 0)), 0xAA, dtype=np.uint8)
    sT = np.full((cols, max(P // 128, 0)), np.nan, dtype=np.float32)
    if P > 0:
        fn = lib.ora_quant_colwise_p2 if pow2 else lib.ora_quant_colwise
        fn(_ptr(x), rows, cols, cols, offs_p, E, _ptr(qT), qT.shape[1], _ptr(sT), sT.shape[1])
    return qT, sT


def requant_colwise(q: np.ndarray, s: np.ndarray, cols: int, offsets: np.ndarray | None = None):
    """Token-axis requantization of saved 1x128 codes q [rows, >= cols] with
    scales s [rows, ceil(cols/128)]: dequantize in fp32, then quant_colwise.
    Returns (qT, sT) in quant_colwise's layout."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    rows = q.shape[0]
    if offsets is None:
        P = _rup(rows, 128)
        offs_p, E = None, 0
    else:
        offsets = np.ascontiguousarray(offsets, dtype=np.int32)
        E = offsets.size - 1
        P = int(padded_offsets(offsets)[-1])
        offs_p = _ptr(offsets)
    qT = np.full((cols, max(P, 0)), 0xAA, dtype=np.uint8)
    sT = np.full((cols, max(P // 128, 0)), np.nan, dtype=np.float32)
    if P > 0:
        lib.ora_requant_colwise(_ptr(q), q.shape[1], _ptr(s), s.shape[1], rows, cols, offs_p, E,
                                _ptr(qT), qT.shape[1], _ptr(sT), sT.shape[1])
    return qT, sT


def e8m0_of_pow2(s: np.ndarray) -> np.ndarray:
    """E8M0 bytes (k + 127) of power-of-two scales 2^k, k in [-127, 127]."""
    s = np.asarray(s, dtype=np.float32)
    m, e = np.frexp(s.astype(np.float64))
    if not np.all(m == 0.5):
        raise ValueError("not a power of two")
    return (e - 1 + 127).astype(np.uint8)


def mx_exponent(amax: float) -> int:
    return int(_load().ora_mx_exponent(float(amax)))


def mx_quant_rows(x: np.ndarray):
    """MXFP8 1x32 along the last axis.  Returns (q [rows, rup(cols,128)] u8,
    e [rows, rup(cols,128)/32] u8 E8M0)."""
    lib = _load()
    x = as_f32(x)
    rows, cols = x.shape
    kp = _rup(cols, 128)
    q = np.full((rows, kp), 0xAA, dtype=np.uint8)
    e = np.full((rows, kp // 32), 0xAA, dtype=np.uint8)
    lib.ora_mx_quant_rows(_ptr(x), rows, cols, cols, _ptr(q), kp, _ptr(e), kp // 32)
    return q, e


def mx_quant_cols(x: np.ndarray):
    """MXFP8 32x1 along the row axis, written transposed.  Returns
    (qT [cols, rup(rows,128)] u8, eT [cols, rup(rows,128)/32] u8)."""
    lib = _load()
    x = as_f32(x)
    rows, cols = x.shape
    kp = _rup(rows, 128)
    qT = np.full((cols, kp), 0xAA, dtype=np.uint8)
    eT = np.full((cols, kp // 32), 0xAA, dtype=np.uint8)
    lib.ora_mx_quant_cols(_ptr(x), rows, cols, cols, _ptr(qT), kp, _ptr(eT), kp // 32)
    return qT, eT


# -------------------------------------------------------- dequantizers
def deq_rowgroups(q: np.ndarray, s: np.ndarray, K: int, group: int = 128) -> np.ndarray:
    lib = _load()
    q = np.ascontiguousarray(q)
    s = np.ascontiguousarray(s, dtype=np.float32)
    rows = q.shape[0]
    out = np.empty((rows, K), dtype=np.float64)
    lib.ora_deq_rowgroups(_ptr(q), q.shape[1], _ptr(s), s.shape[1], rows, K, group, _ptr(out), K)
    return out


def deq_128x128(q: np.ndarray, s: np.ndarray, D: int, C: int) -> np.ndarray:
    lib = _load()
    q = np.ascontiguousarray(q)
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.empty((D, C), dtype=np.float64)
    lib.ora_deq_128x128(_ptr(q), q.shape[1], _ptr(s), s.shape[1], D, C, _ptr(out), C)
    return out


def deq_mx(q: np.ndarray, e: np.ndarray, K: int) -> np.ndarray:
    lib = _load()
    q = np.ascontiguousarray(q)
    e = np.ascontiguousarray(e)
    rows = q.shape[0]
    out = np.empty((rows, K), dtype=np.float64)
    lib.ora_deq_mx(_ptr(q), q.shape[1], _ptr(e), e.shape[1], rows, K, _ptr(out), K)
    return out


def matmul_f64(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """A [M, K] @ B [K, N] in fp64, each sum in ascending k."""
    lib = _load()
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    out = np.empty((M, N), dtype=np.float64)
    lib.ora_matmul_f64(_ptr(A), K, _ptr(B), N, M, N, K, _ptr(out), N)
    return out


# --------------------------------------------------------------- GEMMs
def fprop(xq, xs, wq, ws, C: int, D: int | None = None) -> np.ndarray:
    """Y = X W^T on the dequantized operands (X 1x128, W 128x128)."""
    D = wq.shape[0] if D is None else D
    Xd = deq_rowgroups(xq, xs, C)
    Wd = deq_128x128(wq, ws, D, C)
    return matmul_f64(Xd, Wd.T)


def dgrad(gq, gs, wq, ws, D: int, C: int) -> np.ndarray:
    """dX = dY W, with dY 1x128 along D and W dequantized in its stored
    D x C orientation (no transposed copy needed by the oracle)."""
    Gd = deq_rowgroups(gq, gs, D)
    Wd = deq_128x128(wq, ws, D, C)
    return matmul_f64(Gd, Wd)


def dgrad_from_qT(gq, gs, wqT, ws, D: int, C: int) -> np.ndarray:
    """dX = dY W with W read from its transposed code copy (C x D) and the
    same 128x128 scale grid read transposed."""
    Gd = deq_rowgroups(gq, gs, D)
    WTd = deq_128x128(wqT, np.ascontiguousarray(ws.T), C, D)
    return matmul_f64(Gd, WTd.T)


def wgrad(gqT, gsT, xqT, xsT, K: int) -> np.ndarray:
    """dW = dY^T X with both operands grouped along the token axis
    (contraction length K, padded positions hold zero codes)."""
    GTd = deq_rowgroups(gqT, gsT, K)
    XTd = deq_rowgroups(xqT, xsT, K)
    return matmul_f64(GTd, XTd.T)


def mx_gemm(aq, ae, bq, be, K: int) -> np.ndarray:
    """out[i][j] = sum_k A[i,k] B[j,k], both MX 1x32 along k."""
    Ad = deq_mx(aq, ae, K)
    Bd = deq_mx(bq, be, K)
    return matmul_f64(Ad, Bd.T)


def rel_row_error(y_test: np.ndarray, y_ref: np.ndarray) -> float:
    """max_{i,j} |y_test - y_ref| / ||y_ref[i,:]||_2; a zero reference row
    must be matched exactly (returns inf otherwise)."""
    y_test = np.asarray(y_test, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    norms = np.sqrt(np.sum(y_ref * y_ref, axis=1))
    diff = np.abs(y_test - y_ref)
    worst = 0.0
    zero = norms == 0
    if np.any(zero):
        if np.any(diff[zero] != 0):
            return float("inf")
    nz = ~zero
    if np.any(nz):
        worst = float(np.max(diff[nz] / norms[nz, None]))
    return worst


# ------------------------------------------------ fused producers (f1)
from .fused import (bf16_rne, bf16_rne_from_f64, bf16_to_f32, rmsnorm_bf16,  # noqa: E402
                    rmsnorm_rstd, rmsnorm_sumsq, silu_mul_bf16, silu_table)


def rmsnorm_quant_1x128(x: np.ndarray, w: np.ndarray, eps: float):
    """RMSNorm to bf16, then the 1x128 quantizer.  x and w are float32 or
    bf16 bits.  Returns (q, s, r, y): codes and scales as quant_1x128, the
    per-row r = fl32(1/sqrt(mean(x^2) + eps)) and the bf16 activation bits."""
    y, r = rmsnorm_bf16(as_f32(x), as_f32(w), eps)
    q, s = quant_1x128(y)
    return q, s, r, y


def silu_mul_quant_1x128(gate: np.ndarray, up: np.ndarray):
    """bf16(bf16(silu(gate)) * up), then the 1x128 quantizer.  gate and up
    are bf16 bits.  Returns (q, s, a) with a the bf16 activation bits."""
    a = silu_mul_bf16(gate, up)
    q, s = quant_1x128(a)
    return q, s, a


# ------------------------------------- dequantized backward operands (f4)
def dequant_bf16_rows(q: np.ndarray, s: np.ndarray, cols: int, group: int = 128) -> np.ndarray:
    """bf16 bits of fl32(E4M3(q) * s) for codes grouped along the rows
    (1x128 when group = 128): the exact product (in binary64) rounded to
    binary32, then to bf16 with nearest-even."""
    with np.errstate(over="ignore"):
        return bf16_rne(deq_rowgroups(q, s, cols, group).astype(np.float32))


def dequant_bf16_128x128(q: np.ndarray, s: np.ndarray, D: int, C: int) -> np.ndarray:
    """bf16 bits of fl32(E4M3(q) * s_block) for 128x128-block codes [D, C]."""
    with np.errstate(over="ignore"):
        return bf16_rne(deq_128x128(q, s, D, C).astype(np.float32))


def dequant_bf16_mx(q: np.ndarray, e: np.ndarray, cols: int) -> np.ndarray:
    """bf16 bits of fl32(E4M3(q) * 2^(e - 127)) for MX 1x32 codes."""
    with np.errstate(over="ignore"):
        return bf16_rne(deq_mx(q, e, cols).astype(np.float32))


def bf16_matmul(A_bits: np.ndarray, B_bits: np.ndarray) -> np.ndarray:
    """A [M, K] @ B [K, N] of bf16 bit arrays, in binary64."""
    return matmul_f64(bf16_to_f32(A_bits).astype(np.float64), bf16_to_f32(B_bits).astype(np.float64))
