"""bfloat16 bit patterns (oracle side).

BF16 is the activation precision of the method (Qwen3.5-4B quantization study,
section 2 settings table: 4-bit weights, BF16 inputs).  A bf16 value is the top
16 bits of an IEEE binary32, so widening it is exact.  Narrowing (used for
16-bit restore scales) picks the nearest bf16 value, ties to the even one.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """uint16 (or int16) array of bf16 bit patterns -> float64 array, exactly."""
    b = np.asarray(bits)
    if b.dtype == np.int16:
        b = b.view(np.uint16)
    if b.dtype != np.uint16:
        raise TypeError("expected uint16 bf16 bit patterns")
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_bits(v32):
    """float32 array -> uint16 bf16 bit patterns of the nearest bf16 values.

    Nearest by value, ties to the candidate whose last significand bit is 0;
    +-inf stay infinite and every NaN becomes the quiet NaN 0x7FC0.  The two
    candidates are the bf16 values on either side of v (toward zero: v with its
    low 16 bits cleared; away from zero: the next bf16 up in magnitude), and
    their distances to v are compared in float64, where they are exact.
    """
    v = np.asarray(v32)
    if v.dtype != np.float32:
        raise TypeError("expected float32 values")
    bits = v.view(np.uint32)
    toward = bits & np.uint32(0xFFFF0000)
    away = toward + np.uint32(0x10000)  # next bf16 magnitude (same sign)
    v64 = v.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        lo = toward.view(np.float32).astype(np.float64)
        hi = away.view(np.float32).astype(np.float64)
        # past the largest finite bf16 the next step is infinity, which rounding
        # reaches from the midpoint 2^128 - 2^119 on (IEEE overflow rule)
        hi = np.where(np.isinf(hi) & np.isfinite(v64), np.copysign(2.0 ** 128, v64), hi)
        d_lo = np.abs(v64 - lo)
        d_hi = np.abs(hi - v64)
    lo_even = ((toward >> np.uint32(16)) & np.uint32(1)) == 0
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & lo_even)
    out = np.where(pick_lo, toward, away) >> np.uint32(16)
    out = np.where(np.isinf(v), bits >> np.uint32(16), out)
    out = np.where(np.isnan(v), np.uint32(0x7FC0), out)
    return out.astype(np.uint16)
