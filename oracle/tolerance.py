"""When an output of the linear counts as correct (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The linear is y = W_hat x (Qwen3.5-4B quantization study, section 1, with
BF16 inputs per the section 2 settings table).  The pages fix no output
precision and no error bound; the bound this project holds the kernels to is

    |v - y_ref| <= REL * sum_k |w_hat[n,k] x[m,k]| + ABS,   REL = 2e-3, ABS = 1e-6,

for the value v the kernel accumulates, with y_ref the exact (fp64) product.
Readings:

* an fp32 output is that v itself, so it must satisfy the bound directly;
* a bf16 output is the nearest-even bf16 of such a v.  bf16 keeps 8
  significant bits, so its rounding alone can move a value by up to 2^-8 of
  its magnitude -- more than REL when |y| is close to sum|w_hat x| (rows
  whose products all have one sign).  A bf16 output y is therefore correct
  exactly when some real v within the bound rounds to y: when the interval
  [y_ref - tol, y_ref + tol] meets the set of reals that round to y;
* NaN: an output is NaN exactly where y_ref is NaN (a non-finite weight group
  or a non-finite activation row, see oracle/linear.py);
* infinities: +-inf is correct when the interval reaches the values that
  round to it (at least halfway between the largest finite value and 2^128).

Every value used here (bf16 and fp32 values, their neighbours and midpoints)
is exact in float64.
"""

import numpy as np

REL_TOL = 2e-3
ABS_TOL = 1e-6

# (storage dtype, exponent-field shift, sign bit, bit pattern of +inf)
_FORMATS = {
    "bf16": (np.uint16, np.uint32(16), np.uint32(0x8000), np.uint32(0x7F80)),
    "f32": (np.uint32, np.uint32(0), np.uint32(0x80000000), np.uint32(0x7F800000)),
}


def _value(mag_bits, shift):
    """float64 value of non-negative bit patterns (as uint32 magnitudes) of the format."""
    return (mag_bits.astype(np.uint32) << shift).view(np.float32).astype(np.float64)


def rounding_interval(bits, fmt):
    """[lo, hi]: the reals that round (nearest, ties to even) to the finite
    values with these bit patterns, as float64 arrays (closed at both ends;
    non-finite patterns are read as the largest finite magnitude)."""
    dtype, shift, sign_bit, inf_bits = _FORMATS[fmt]
    b = np.asarray(bits).astype(np.uint32)
    mag = np.minimum(b & (sign_bit - np.uint32(1)), inf_bits - np.uint32(1))  # finite patterns only
    neg = (b & sign_bit) != 0
    v = _value(mag, shift)
    # the next magnitude up (past the largest finite value: 2^128) and down
    top = inf_bits - np.uint32(1)  # the largest finite magnitude
    up = np.where(mag >= top, 2.0 ** 128, _value(np.minimum(mag + np.uint32(1), top), shift))
    dn = np.where(mag == 0, -_value(np.ones_like(mag), shift), _value(np.maximum(mag, np.uint32(1)) - np.uint32(1), shift))
    gap_up = (up - v) / 2.0
    gap_dn = (v - dn) / 2.0
    lo = np.where(neg, -(v + gap_up), v - gap_dn)
    hi = np.where(neg, -(v - gap_dn), v + gap_up)
    return lo, hi


def admissible(y_bits, y_ref, absdot, fmt, rel=REL_TOL, abs_=ABS_TOL):
    """Elementwise: is the output with these bit patterns (uint16 bf16 or uint32
    fp32) a correct result for the exact value y_ref (float64), given
    absdot = sum_k |w_hat x|?  See the module docstring."""
    dtype, shift, sign_bit, inf_bits = _FORMATS[fmt]
    b = np.asarray(y_bits)
    if b.dtype != dtype:
        raise TypeError(f"{fmt} outputs must be {np.dtype(dtype).name} bit patterns")
    b = b.astype(np.uint32)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    tol = rel * np.asarray(absdot, dtype=np.float64) + abs_
    mag = b & (sign_bit - np.uint32(1))
    neg = (b & sign_bit) != 0
    is_nan = mag > inf_bits
    is_inf = mag == inf_bits
    ref_nan = np.isnan(y_ref) | np.isnan(tol)
    with np.errstate(invalid="ignore"):
        lo, hi = rounding_interval(np.where(is_nan | is_inf, 0, b).astype(dtype), fmt)
        a, z = y_ref - tol, y_ref + tol
        finite_ok = (a <= hi) & (z >= lo)
        # halfway between the largest finite value and 2^128: rounds to infinity
        big = (_value(inf_bits - np.uint32(1), shift) + 2.0 ** 128) / 2.0
        inf_ok = np.where(neg, a <= -big, z >= big)
    ok = np.where(is_inf, inf_ok, finite_ok)
    return np.where(ref_nan, is_nan, ok & ~is_nan)


def worst_ratio(y, y_ref, absdot, rel=REL_TOL, abs_=ABS_TOL):
    """max |y - y_ref| / tol over the non-NaN references (a diagnostic)."""
    y = np.asarray(y, dtype=np.float64)
    ok = ~np.isnan(y_ref)
    if not ok.any():
        return 0.0
    with np.errstate(invalid="ignore"):
        r = np.abs(y[ok] - y_ref[ok]) / (rel * absdot[ok] + abs_)
    return float(np.nanmax(r)) if r.size else 0.0
