"""Number formats used by the oracle: bfloat16, OCP FP8 E4M3 (e4m3fn) and the
OCP Microscaling MXFP4 weight format (FP4 E2M1 elements, E8M0 block scales).

TEST INFRASTRUCTURE ONLY.  See ``oracle/__init__.py``.

bfloat16 is the upper 16 bits of an IEEE binary32 value (8 significant bits,
binary32's exponent range).  E4M3 here is the OCP 8-bit floating point format
E4M3 ("FN"): sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, S.1111.111 is NaN, largest finite magnitude 448, smallest
subnormal 2^-9.  Both encoders round to nearest, ties to even; the E4M3
encoder saturates finite values beyond 448 to +-448 (the reading recorded for
the FP8 workload: an fp8 grouped GEMM stores finite codes only).
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------- bfloat16

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, ONE rounding to nearest even.

    Writes v = m * 2**e with 0.5 <= |m| < 1, keeps 8 significant bits of m by
    rounding m * 2**8 to the nearest integer (ties to even, exact in float64)
    and rescales.  Below binary32's normal range the quantum stays 2**-133.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    e = np.maximum(e, -125)  # subnormal range: fixed quantum 2**(-125-8)
    q = np.rint(np.ldexp(v, 8 - e))  # integer significand, |q| <= 256
    r = np.ldexp(q, e - 8)
    if np.any(np.abs(r) > 3.3895313892515355e38):
        raise OverflowError("value beyond the bfloat16 range")
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def f32_to_bf16(v: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (exact input, one rounding)."""
    return f64_to_bf16(np.asarray(v, dtype=np.float32).astype(np.float64))


# ----------------------------------------------------------------------------- E4M3

def _e4m3_from_bits(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> float64, from the bit-field definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    sub = man / 8.0 * 2.0 ** -6
    nor = (1.0 + man / 8.0) * np.ldexp(1.0, (exp - 7).astype(np.int64))
    val = sign * np.where(exp == 0, sub, nor)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# the value of every one of the 256 codes, from the bit-field definition above
_E4M3_TABLE = _e4m3_from_bits(np.arange(256, dtype=np.uint8))


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> float64: the bit-field definition's value of each code
    (looked up in the table of all 256 codes, so large weight matrices decode quickly)."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


_POS_CODES = np.arange(0x7F, dtype=np.uint8)  # 0x00..0x7E: every non-negative finite code
_POS_VALUES = e4m3_decode(_POS_CODES)  # strictly increasing


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float -> E4M3 codes: the nearest finite code, ties to the even code, |v| > 448 -> +-448.

    Finds the two neighbouring representable magnitudes in the table of all
    finite codes and picks the nearer one.  No NaN input is expected.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("NaN input to e4m3_encode")
    a = np.minimum(np.abs(v), 448.0)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _POS_VALUES[hi], hi, code).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


# ----------------------------------------------------------------------------- MXFP4

def _e2m1_from_bits(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes (low 4 bits) -> float64, from the bit-field definition of the OCP
    Microscaling Formats (MX) v1.0 spec: sign bit, 2 exponent bits with bias 1, 1
    mantissa bit, exponent field 0 is subnormal (0 or 0.5); no infinities or NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    exp = (c >> 1) & 0x3
    man = c & 0x1
    val = np.where(exp == 0, man * 0.5, (1.0 + man / 2.0) * np.ldexp(1.0, (exp - 1).astype(np.int64)))
    return sign * val


_E2M1_TABLE = _e2m1_from_bits(np.arange(16, dtype=np.uint8))  # the 16 codes, from the definition above


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes (low 4 bits) -> float64: the bit-field definition's value of each code
    (looked up in the table of all 16 codes)."""
    return _E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & np.uint8(0xF)]


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale codes -> 2^(code - 127) as float64 (255 is NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def mxfp4_dequant(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """An MXFP4 matrix -> float64 (exact): packed [rows, cols/2] holds two E2M1 codes per byte
    (the even column in the low nibble), scales [rows, cols/32] one E8M0 code per row and
    32 consecutive columns."""
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = p & 0xF
    codes[:, 1::2] = p >> 4
    return e2m1_decode(codes) * np.repeat(e8m0_decode(scales), 32, axis=1)
