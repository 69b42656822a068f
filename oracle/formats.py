"""Number formats used by NVFP4: BF16, FP8 E4M3 (block scales), FP4 E2M1 (elements).

TEST INFRASTRUCTURE ONLY (see the package docstring).

*The 4-bitter Lesson*, section "Baseline: A starting recipe with stable training
dynamics": NVFP4 stores 4-bit floating-point values in blocks of 16, each block
carrying an FP8 E4M3 scale, with one FP32 scale for the whole tensor.

The encodings below are written from the format definitions:

* FP4 E2M1 (OCP MX v1.0, FP4 element type): 1 sign bit, 2 exponent bits with
  bias 1, 1 mantissa bit, no infinity or NaN.  The eight magnitudes are
  0, 0.5, 1, 1.5, 2, 3, 4, 6 and the 3-bit magnitude field is their index.
* FP8 E4M3 (OCP OFP8): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
  subnormals m * 2^-9, no infinities, S.1111.111 is NaN, largest finite 448.
* BF16: the upper 16 bits of an IEEE binary32.

Rounding.  *The 4-bitter Lesson*, section "Improving Gradient Stability"
(footnote 6) writes quantisation as clip(round(w/s), qmin, qmax).  The pages do
not name the rounding mode; the reading taken here is round-to-nearest with
ties to the even code, and clipping to the largest finite magnitude.
"""

from __future__ import annotations

import numpy as np

# Magnitudes of FP4 E2M1, indexed by the 3-bit exponent|mantissa field.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0
E4M3_NAN_CODE = 0x7F


# ----------------------------------------------------------------------------- BF16

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float32 values (exact: the bits become the
    upper half of a binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns, round to nearest, ties to even.

    The BF16 value nearest to x is found by comparing x with its two BF16
    neighbours (truncation and truncation + 1 ulp) in FP64, which holds every
    binary32 and every midpoint between BF16 values exactly.  NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lo = (u >> np.uint32(16)).astype(np.uint32)            # toward zero
    hi = lo + np.uint32(1)                                  # away from zero
    lo_v = (lo << np.uint32(16)).view(np.float32).astype(np.float64)
    with np.errstate(invalid="ignore"):
        hi_v = (hi << np.uint32(16)).view(np.float32).astype(np.float64)
    # above the largest finite BF16 the next "value" is 2^128 (IEEE overflow
    # rounds as if the exponent range were unbounded, then becomes infinity)
    hi_v = np.where((hi & np.uint32(0x7FFF)) == 0x7F80, np.copysign(2.0 ** 128, hi_v), hi_v)
    xv = x.astype(np.float64)
    d_lo = np.abs(xv - lo_v)
    with np.errstate(invalid="ignore"):
        d_hi = np.abs(hi_v - xv)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & np.uint32(1)) == 1))
    out = np.where(pick_hi, hi, lo).astype(np.uint32)
    nan = np.isnan(x)
    out = np.where(nan, np.uint32(0x7FC0) | (lo & np.uint32(0x8000)), out)
    return out.astype(np.uint16)


# ----------------------------------------------------------------------------- E2M1

def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit codes (bit 3 = sign, bits 2..0 = magnitude index) -> FP64 values."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[c & 0x7]
    return np.where((c & 0x8) != 0, -mag, mag)


def _nearest_even(values: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the entry of the ascending ``table`` nearest to each of
    ``values`` (FP64, non-negative); on an exact tie between two neighbours the
    even index wins.  Values above the last entry map to the last entry."""
    v = np.asarray(values, dtype=np.float64)
    hi = np.searchsorted(table, v, side="left")           # first entry >= v
    hi = np.minimum(hi, len(table) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = np.abs(v - table[lo])
    d_hi = np.abs(table[hi] - v)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(take_hi, hi, lo)
    # v at or below the first entry, or at or above the last, has one candidate
    # (for huge v the FP64 distances to the last two entries can compare equal)
    idx = np.where(v <= table[0], 0, idx)
    idx = np.where(v >= table[-1], len(table) - 1, idx)
    return idx.astype(np.int64)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """FP32 values -> E2M1 codes: round |v| to the nearest magnitude (ties to
    the even index, saturating at 6), sign bit copied from v (so -0 and
    negatives that round to zero give code 0x8)."""
    v = np.asarray(v, dtype=np.float32)
    if np.isnan(v).any():
        raise ValueError("E2M1 encode of NaN is outside the method's contract")
    a = np.abs(v.astype(np.float64))
    idx = _nearest_even(a, E2M1_MAGNITUDES)
    sign = np.signbit(v).astype(np.uint8) << 3
    return (sign | idx.astype(np.uint8)).astype(np.uint8)


# ----------------------------------------------------------------------------- E4M3

def e2m1_encode_sr(v: np.ndarray, u24: np.ndarray) -> np.ndarray:
    """Stochastic rounding onto the E2M1 grid (the pretraining recipe's gradient
    rounding, *The 4-bitter Lesson*, section "Why is the NVFP4 pretraining recipe
    not sufficient for RL?").  |v| >= 6 saturates to 6.  Otherwise, with lo and hi
    the grid neighbours of |v|, the magnitude rounds up to hi exactly when
    u24 * 2^-24 < (|v| - lo) / (hi - lo), so the probability of rounding up is that
    fraction (to 24 bits) and the rounding is unbiased.  The sign comes from v.
    Every quantity here is exact in FP64 (and in FP32: |v| - lo is exact because
    lo = 0 or hi <= 2 lo, and the grid gaps are powers of two)."""
    v = np.asarray(v, dtype=np.float32)
    u24 = np.asarray(u24, dtype=np.uint32)
    a = np.minimum(np.abs(v).astype(np.float64), E2M1_MAX)
    i = np.searchsorted(E2M1_MAGNITUDES, a, side="right") - 1     # largest grid value <= a
    lo = E2M1_MAGNITUDES[i]
    top = i == len(E2M1_MAGNITUDES) - 1
    gap = np.where(top, 1.0, E2M1_MAGNITUDES[np.minimum(i + 1, len(E2M1_MAGNITUDES) - 1)] - lo)
    frac = (a - lo) / gap
    up = (~top) & (u24.astype(np.float64) * 2.0 ** -24 < frac)
    mag = (i + up).astype(np.uint8)
    return (np.signbit(v).astype(np.uint8) << 3 | mag).astype(np.uint8)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 byte -> FP64 value (closed form); 0x7F / 0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == E4M3_NAN_CODE, np.nan, mag)
    return np.where((c & 0x80) != 0, -mag, mag)


def e4m3_finite_nonneg() -> np.ndarray:
    """The 127 non-negative finite E4M3 values, ascending; index == code."""
    return e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))


_E4M3_TABLE = e4m3_finite_nonneg()


def e4m3_encode(t: np.ndarray) -> np.ndarray:
    """Non-negative FP32 -> E4M3 byte: values at or above 448 saturate to 448
    (code 0x7E); otherwise the nearest finite value, ties to the even code."""
    t = np.asarray(t, dtype=np.float32)
    if (t < 0).any() or np.isnan(t).any():
        raise ValueError("block scales are non-negative and finite")
    tv = np.minimum(t.astype(np.float64), E4M3_MAX)
    return _nearest_even(tv, _E4M3_TABLE).astype(np.uint8)


# ----------------------------------------------------------------------------- FP32 helpers

def f32(x) -> np.ndarray:
    """Round FP64 values to the nearest FP32 (ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_div(a, b) -> np.ndarray:
    """Correctly rounded FP32 quotient of FP32 operands.

    The quotient is formed in FP64 and rounded once more to FP32; because FP64
    carries more than 2*24+2 bits, this double rounding equals the correctly
    rounded FP32 quotient (Figueroa, "When is double rounding innocuous?",
    SIGNUM 1995)."""
    return f32(np.asarray(a, np.float32).astype(np.float64) / np.asarray(b, np.float32).astype(np.float64))


def f32_mul(a, b) -> np.ndarray:
    """Correctly rounded FP32 product of FP32 operands (the FP64 product of two
    FP32 values is exact, so one rounding to FP32 is the IEEE result)."""
    return f32(np.asarray(a, np.float32).astype(np.float64) * np.asarray(b, np.float32).astype(np.float64))
