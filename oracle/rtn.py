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

Readings where the pages are silent (each one also listed in the design doc):

* range and scale: a = max |w| over the group, d = fl32(a / 7) (symmetric
  min/max; the largest magnitude maps to code +-7);
* codes span [-8, 7] (16 values) and the division is by the *stored* fp32 d,
  t = fl32(w / d), IEEE round-to-nearest-even, no flush of subnormals;
* "round" moves to the nearest integer with ties away from zero;
* a group holding a NaN or an infinity gets d = NaN (bit pattern 0x7FC00000)
  and all codes 0; a group whose scale is zero (all-zero group, or a/7
  underflowing to 0) gets all codes 0.
"""

import numpy as np

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


def rtn_quantize_ref(W):
    """Quantize a weight matrix group by group.

    W: float32 array [N, K] (N outputs, K inputs), K a positive multiple of 128.
    Returns (q, d): q int8 [N, K] holding codes in [-8, 7] (canonical order),
    d float32 [N, K/128] holding one restore scale per (row, group).
    """
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
    usable = finite & (d != 0)

    # Step 3: codes q = clip(round(w / d) + z, qmin, qmax), z = 0, dividing by
    # the stored fp32 scale.
    safe_d = np.where(usable, d, np.float32(1.0)).astype(np.float32)
    with np.errstate(all="ignore"):
        t = (Wg / safe_d[:, :, None]).astype(np.float32)
    q = np.clip(_round_half_away(t), QMIN, QMAX)
    q[~usable] = 0
    return q.reshape(N, K).astype(np.int8), d
