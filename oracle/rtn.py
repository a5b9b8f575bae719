"""Round-to-nearest symmetric INT4 group quantizer (oracle, fp32).

Follows the group-quantization equation of the Qwen3.5-4B quantization study,
section 1 ("what was compressed"):

    q = clip(round(w / d) + z, qmin, qmax),        w_hat = d * (q - z)

with the symbols as that section's table defines them: q is one of the 16
codes a 4-bit slot can hold, d is the restore scale shared by one group, z is
the zero point, which a symmetric scheme does not search (so z = 0 here).  A
group is 128 consecutive weights of one row along the input direction
(section 1, the 2560x9216 example: 72 groups per row).  Section 2's settings
table fixes RTN at group size 128 with a symmetric range taken from the
group's min/max and no clipping-ratio search, and notes RTN uses no
calibration input.

Readings where the pages are silent:

* range and scale: a = max |w| over the group, d = fl32(a / 7) (symmetric
  min/max; the largest magnitude maps to code +-7);
* codes span [-8, 7] (16 values) and the division is by the *stored* fp32 d,
  t = fl32(w / d), IEEE round-to-nearest-even, no flush of subnormals;
* "round" moves to the nearest integer with ties away from zero;
* a group holding a NaN or an infinity gets d = NaN (bit pattern 0x7FC00000)
  and all codes 0; a group whose scale is zero (all-zero group, or a/7
  underflowing to 0) gets all codes 0.

16-bit scales (the study's checkpoint sizes imply about two bytes per group;
the pages do not name the format): d is computed in fp32 as above, then
stored as the nearest bf16 value (ties to even, NaN -> 0x7FC0), and the
codes divide by that stored value widened back to fp32: t = fl32(w / d16).
bf16 keeps fp32's exponent range, so no scale overflows or needs clamping.
"""

import numpy as np

from .bf16 import f32_to_bf16_bits

GROUP = 128
QMIN = -8
QMAX = 7
NAN_BITS = 0x7FC00000


def _nan_f32():
    return np.array([NAN_BITS], dtype=np.uint32).view(np.float32)[0]


def _round_half_away(t32):
    """Nearest integer to fp32 values, ties away from zero.

    Done in fp64, where t + 0.5 is exact for every fp32 t, so there is no
    double rounding.  (np.round would round ties to even.)
    """
    t = t32.astype(np.float64)
    return np.trunc(t + np.copysign(0.5, t))


def rtn_quantize_ref(W, scale_dtype="f32"):
    """Quantize a weight matrix group by group.

    W: float32 array [N, K] (N outputs, K inputs), K a positive multiple of 128.
    Returns (q, d): q int8 [N, K] holding codes in [-8, 7] (canonical order),
    d [N, K/128] holding one restore scale per (row, group): float32 values
    for scale_dtype "f32", uint16 bf16 bit patterns for "bf16".
    """
    if scale_dtype not in ("f32", "bf16"):
        raise ValueError("scale_dtype must be 'f32' or 'bf16'")
    W = np.asarray(W)
    if W.dtype != np.float32 or W.ndim != 2:
        raise TypeError("W must be a 2-D float32 array")
    N, K = W.shape
    if K <= 0 or K % GROUP:
        raise ValueError("K must be a positive multiple of 128")
    G = K // GROUP
    Wg = W.reshape(N, G, GROUP)

    # Step 1: the group's range.  Symmetric min/max: the largest magnitude.
    finite = np.isfinite(Wg).all(axis=2)
    with np.errstate(invalid="ignore"):
        a = np.abs(Wg).max(axis=2).astype(np.float32)

    # Step 2: the restore scale d, so that +-a maps to code +-7 (fp32 IEEE divide).
    with np.errstate(all="ignore"):
        d = (a / np.float32(7.0)).astype(np.float32)
    d[~finite] = _nan_f32()
    if scale_dtype == "bf16":
        # Step 2b: the stored scale is the nearest bf16; the codes use it.
        d_bits = f32_to_bf16_bits(d)
        d = (d_bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    usable = finite & (d != 0)

    # Step 3: codes q = clip(round(w / d) + z, qmin, qmax), z = 0, dividing by
    # the stored scale (widened to fp32).
    safe_d = np.where(usable, d, np.float32(1.0)).astype(np.float32)
    with np.errstate(all="ignore"):
        t = (Wg / safe_d[:, :, None]).astype(np.float32)
    q = np.clip(_round_half_away(t), QMIN, QMAX)
    q[~usable] = 0
    q = q.reshape(N, K).astype(np.int8)
    return (q, d_bits) if scale_dtype == "bf16" else (q, d)
