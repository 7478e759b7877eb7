"""Quantised key/value cache for the CPU oracle (test infrastructure only).

The pages reach long contexts in small memory with a quantised KV cache (Lucebox-Hub
review, section "2. DFlash", 256K context with a compressed cache); they do not define a
format, so this one is self-defined and written to be exact where it matters:

* Codes: OCP 8-bit floating point E4M3 (1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits; subnormals at exponent field 0; largest finite value 448; the pattern
  S.1111.111 is NaN and never produced here). Encoding rounds to nearest, ties to even.
* Scale: one power of two per (token, KV head) row of D values: the smallest 2^e with
  max|x| <= 448 * 2^e (2^0 for an all-zero row). x / 2^e is then exact and within range,
  so a code is the E4M3 rounding of an exactly known number.
* Dequantisation: code value * 2^e, exactly representable in bfloat16 (at most 4
  significant bits, exponent well inside range), so an attention kernel that widens codes
  to bf16 sees exactly the values this oracle uses.
"""

from __future__ import annotations

import math

import numpy as np

from .tree_verify import bf16_bits_to_f64

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes (uint8). NaN codes decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def _e4m3_table():
    codes = np.arange(0, 0x7F, dtype=np.uint8)          # non-negative finite codes 0 .. 0x7E
    return codes, e4m3_decode(codes)


def e4m3_encode(x) -> np.ndarray:
    """Round float64 values with |x| <= 448 to the nearest E4M3 code, ties to the even code.

    Written as a search over the 127 non-negative finite code values (plain and slow): the
    nearest value wins; at an exact midpoint the code with an even mantissa field (lowest
    bit 0) wins."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or np.any(~np.isfinite(x)):
        raise ValueError("values must be finite with |x| <= 448")
    codes, vals = _e4m3_table()
    a = np.abs(x).ravel()
    idx = np.searchsorted(vals, a)                        # vals[idx-1] < a <= vals[idx]
    hi = np.clip(idx, 0, len(vals) - 1)
    lo = np.clip(idx - 1, 0, len(vals) - 1)
    d_hi, d_lo = vals[hi] - a, a - vals[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    out = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    out = np.where(a == 0, 0, out).astype(np.uint8)
    sign = (x.ravel() < 0) & (out != 0)
    out = out | np.where(sign, 0x80, 0).astype(np.uint8)
    return out.reshape(x.shape)


def row_scale_exponent(amax: float) -> int:
    """Smallest e with amax <= 448 * 2^e (0 for amax == 0), by exact exponent arithmetic."""
    if amax == 0:
        return 0
    m, k = math.frexp(amax)            # amax = m * 2^k, 0.5 <= m < 1; 448 = 0.875 * 2^9
    return k - 9 if m <= 0.875 else k - 8


def row_scale_exponents(amax) -> np.ndarray:
    """row_scale_exponent over an array of row maxima (frexp is exact in float64)."""
    amax = np.asarray(amax, dtype=np.float64)
    m, k = np.frexp(amax)
    e = np.where(m <= 0.875, k - 9, k - 8)
    return np.where(amax == 0, 0, e).astype(np.int32)


def quantize_kv(bits, chunk_rows: int = 1 << 16) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits [T, H, D] -> (E4M3 codes uint8 [T, H, D], scale exponents int32 [T, H]).

    Rows are independent: each is scaled by 2^-e (exact) and encoded; tokens are processed
    in chunks only to bound memory."""
    bits = np.asarray(bits)
    T, H, D = bits.shape
    exps = np.zeros((T, H), dtype=np.int32)
    codes = np.zeros((T, H, D), dtype=np.uint8)
    for t0 in range(0, T, chunk_rows):
        x = bf16_bits_to_f64(bits[t0:t0 + chunk_rows])
        e = row_scale_exponents(np.abs(x).max(axis=2))
        exps[t0:t0 + chunk_rows] = e
        codes[t0:t0 + chunk_rows] = e4m3_encode(np.ldexp(x, -e[..., None].astype(np.int64)))
    return codes, exps


def dequantize_kv(codes, exps) -> np.ndarray:
    """float64 [T, H, D] = code value * 2^exponent."""
    return np.ldexp(e4m3_decode(codes), np.asarray(exps, dtype=np.int64)[..., None])


# ---------------------------------------------------------------- 4-bit (MX-style) cache
#
# A sub-8-bit cache in the block structure of the OCP Microscaling (MX) formats: blocks of
# 32 consecutive values of a row share one power-of-two scale, and each value is an OCP
# FP4 E2M1 element (1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit; magnitudes
# 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN). Self-defined where the pages are
# silent, and exact where it matters:
#
# * Scale: per block the smallest 2^e with max|x| <= 6 * 2^e (2^0 for an all-zero block),
#   clamped to e in [-125, 125] (so that every element value times 2^e is a finite bf16
#   and 2^e a normal float32). The MX specification instead takes floor(log2 max|x|) - 2
#   and lets the largest elements clip; the smallest scale that fits clips nothing.
# * Element: x * 2^-e (exact) rounded to the nearest E2M1 value, ties to the even code
#   (mantissa bit 0); magnitudes above 6 (possible only where e was clamped) saturate to 6;
#   a negative value that rounds to zero is coded +0.
# * Packing: element 2j of a row in the low nibble of byte j, element 2j + 1 in the high
#   nibble; scales as int8 exponents [T, H, D / 32].
# * Dequantisation: decode(code) * 2^e, exactly representable in bfloat16.

MX4_BLOCK = 32
E2M1_MAX = 6.0
MX4_EXP_MIN = -125
MX4_EXP_MAX = 125


def e2m1_decode(codes) -> np.ndarray:
    """float64 values of E2M1 codes (integers 0 .. 15)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    val = np.where(e == 0, m * 0.5, (1 + m / 2.0) * 2.0 ** (e - 1))
    return s * val


def e2m1_encode(y) -> np.ndarray:
    """Nearest E2M1 code (uint8 0 .. 15) of float64 values, ties to the even code,
    saturating at +-6; -0 and negative values rounding to zero give code 0.

    The same search as e4m3_encode, over the eight non-negative code values: the nearest
    value wins; at an exact midpoint the code with mantissa bit 0 wins."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)):
        raise ValueError("values must be finite")
    codes = np.arange(8, dtype=np.uint8)
    vals = e2m1_decode(codes)                                 # ascending
    a = np.minimum(np.abs(y).ravel(), E2M1_MAX)
    idx = np.searchsorted(vals, a)                            # vals[idx-1] < a <= vals[idx]
    hi = np.clip(idx, 0, 7)
    lo = np.clip(idx - 1, 0, 7)
    d_hi, d_lo = vals[hi] - a, a - vals[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    pick = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    sign = (y.ravel() < 0) & (pick != 0)
    return (pick | np.where(sign, 0x8, 0).astype(np.uint8)).reshape(y.shape)


def mx4_block_exponent(amax: float) -> int:
    """Smallest e with amax <= 6 * 2^e (0 for amax == 0), clamped to [-125, 125]; by exact
    exponent arithmetic (6 = 0.75 * 2^3)."""
    if amax == 0:
        return 0
    m, k = math.frexp(amax)            # amax = m * 2^k, 0.5 <= m < 1
    e = k - 3 if m <= 0.75 else k - 2
    return min(max(e, MX4_EXP_MIN), MX4_EXP_MAX)


def mx4_block_exponents(amax) -> np.ndarray:
    """mx4_block_exponent over an array of block maxima (frexp is exact in float64)."""
    amax = np.asarray(amax, dtype=np.float64)
    m, k = np.frexp(amax)
    e = np.clip(np.where(m <= 0.75, k - 3, k - 2), MX4_EXP_MIN, MX4_EXP_MAX)
    return np.where(amax == 0, 0, e).astype(np.int64)


def quantize_kv_mx4(bits) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits [T, H, D] -> (packed E2M1 codes uint8 [T, H, D / 2], block exponents int8
    [T, H, D / 32]). Each block is scaled by 2^-e (exact) and encoded."""
    bits = np.asarray(bits)
    T, H, D = bits.shape
    x = bf16_bits_to_f64(bits).reshape(T, H, D // MX4_BLOCK, MX4_BLOCK)
    amax = np.abs(x).max(axis=3)
    exps = mx4_block_exponents(amax)
    codes = e2m1_encode(np.ldexp(x, -exps[..., None])).reshape(T, H, D)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, exps.astype(np.int8)


def dequantize_kv_mx4(packed, exps) -> np.ndarray:
    """float64 [T, H, D] = decode(code) * 2^(exponent of its block)."""
    packed = np.asarray(packed, dtype=np.uint8)
    T, H, D2 = packed.shape
    codes = np.empty((T, H, 2 * D2), dtype=np.uint8)
    codes[..., 0::2] = packed & 0xF
    codes[..., 1::2] = packed >> 4
    e = np.repeat(np.asarray(exps, dtype=np.int64), MX4_BLOCK, axis=2)
    return np.ldexp(e2m1_decode(codes), e)
