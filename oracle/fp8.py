"""FP8 (E4M3) KV-cache elements: the encoding, the decoding and the
quantisation of bf16 K/V rows.  TEST INFRASTRUCTURE ONLY (see the package
docstring).

"The pantry of pigeonholes", the knobs table and "With KV quantisation": an
FP8 KV cache stores each K/V element in one byte instead of two, which halves
the bytes per token.  The pages name no format or scaling.  Readings:

  * The element format is E4M3 in its finite-only ("fn") form: 1 sign bit,
    4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
    subnormals m * 2^-9; there is no infinity; S.1111.111 is NaN; the
    largest finite magnitude is 1.75 * 2^8 = 448.
  * One fp32 scale per cache (K and V each), as a single knob implies: the
    stored code is E4M3(x * r) with r = fp32(1 / scale) and the product
    rounded to fp32; its value is decode(code) * scale.
  * Rounding to E4M3 is to nearest, ties to even; magnitudes above 448
    (infinities included) saturate to 448 with their sign; NaN stays NaN.

Everything below is written from the format's definition; pins compare it
with torch's float8_e4m3fn conversion and with the format's fixed points.
"""

from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F
MIN_NORMAL_EXP = -6        # 2^-6: smallest normal magnitude
SUB_STEP_EXP = -9          # subnormal spacing 2^-9


def decode(codes) -> np.ndarray:
    """E4M3 codes (uint8 array) -> exact values (float64; NaN codes -> NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** SUB_STEP_EXP, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def _round_half_even(x: np.ndarray) -> np.ndarray:
    """Nearest integer, ties to even (x float64, exact for our magnitudes)."""
    f = np.floor(x)
    r = x - f
    up = (r > 0.5) | ((r == 0.5) & (np.mod(f, 2.0) == 1.0))
    return f + up


def encode(values) -> np.ndarray:
    """fp32 values -> E4M3 codes (uint8), round to nearest even, saturating.

    Every fp32 value is exact in float64, so the arithmetic below (powers of
    two and a rounding of a value with few significant bits) is exact."""
    x = np.asarray(values, dtype=np.float32).astype(np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    out = np.zeros(x.shape, dtype=np.int64)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, MAX_FINITE))       # saturate (inf too)
    sub = a < 2.0 ** MIN_NORMAL_EXP
    # subnormal range: a multiple of 2^-9, possibly rounding up to 2^-6 (code 8)
    q_sub = _round_half_even(a * 2.0 ** -SUB_STEP_EXP)
    # normal range: a = 2^e * (1 + f), three fraction bits kept
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(sub, 1.0, a)))
    # log2 of an exact power of two is exact; guard the floor against a
    # last-place error just below one
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    e = np.where(np.exp2(e) > a, e - 1, e)
    mant = _round_half_even((a / np.exp2(e) - 1.0) * 8.0)      # 0..8
    carry = mant == 8
    e = np.where(carry, e + 1, e)
    mant = np.where(carry, 0, mant)
    q_norm = ((e + 7) * 8 + mant).astype(np.int64)
    out = np.where(sub, q_sub.astype(np.int64), q_norm)
    out = np.minimum(out, 0x7E)                                 # 448 after rounding
    out = np.where(nan, NAN_CODE, out)
    out = out | np.where(neg, 0x80, 0)
    return out.astype(np.uint8)


def reciprocal(scale: float) -> np.float32:
    """fp32(1 / scale) with both operands fp32 (one IEEE division)."""
    return np.float32(1.0) / np.float32(scale)


def quantize_bf16(bits, scale: float) -> np.ndarray:
    """bf16 bit patterns -> E4M3 codes of value * fp32(1 / scale) (product
    rounded to fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    x = b.view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (x * reciprocal(scale)).astype(np.float32)
    return encode(y)


def dequantize(codes, scale: float) -> np.ndarray:
    """E4M3 codes -> value * scale in float64."""
    return decode(codes) * np.float64(np.float32(scale))
