"""GPTQ: group-wise INT4 codes chosen column by column with error feedback (oracle, fp64).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Qwen3.5-4B quantization study, section 2 ("what each method fixed"): GPTQ keeps
RTN's storage (symmetric INT4, group 128, the same code and scale arrays), and
instead of rounding every weight independently it quantizes one input column
at a time and corrects the columns not yet quantized, using a Hessian built
from calibration inputs.  The settings table fixes a damping of 0.01 (times the
mean of the Hessian's diagonal), blocks of 128 columns and no column
reordering; the section's output-error equation Delta y = (W_hat - W) x is the
quantity the procedure keeps small.

The update rule itself is the published GPTQ algorithm (Frantar, Ashkboos,
Hoefler and Alistarh, "GPTQ: accurate post-training quantization for
generative pre-trained transformers", 2022), restated here:

* H = (2/T) X^T X over the T calibration rows x_t (K x K), damped,
  H' = H + lambda I, lambda = 0.01 * mean(diag H);
* U is the upper-triangular factor of the inverse, H'^-1 = U^T U;
* for each column j in order: quantize w_j, err = (w_j - w_hat_j) / U[j, j],
  and subtract err * U[j, k] from every later column k.  Within a block of
  128 columns this happens column by column; the columns after the block
  receive the block's accumulated correction in one product (E U[block, rest]).
  In exact arithmetic this equals re-solving, after each column, for the
  remaining columns that minimise (w - w_orig)^T H' (w - w_orig) given every
  column fixed so far -- the property tests/pins.py checks by brute force.

Readings where the pages and the paper leave a step open:

* the group's scale is taken when the group starts, from its current
  (already corrected) weights, by the RTN rule d = fl32(max |fl32(w)| / 7);
  the groups coincide with the 128-column blocks;
* the code decision follows RTN exactly: t = fl32(fl32(w) / d), round half
  away from zero, clamp to [-8, 7]; w_hat = d * q; a group whose scale is 0
  gets codes 0;
* a column whose calibration inputs are all zero (diag H = 0) gets
  H_jj = 1 before damping, so the factorization exists; its weights are kept;
* weights and calibration inputs must be finite;
* with 16-bit scales (the optional storage of RTN, same rule): the group's
  scale is stored as the nearest bf16 of the fp32 scale, and the codes and
  the corrections use that stored value, widened back to fp32.
"""

import numpy as np

from .bf16 import bf16_bits_to_f64, f32_to_bf16_bits
from .rtn import GROUP, QMAX, QMIN

DAMP = 0.01


def gptq_hessian_ref(x_bits):
    """H = (2/T) X^T X in fp64 from bf16 calibration rows [T, K] (uint16 bit patterns)."""
    X = bf16_bits_to_f64(x_bits)
    if not np.isfinite(X).all():
        raise ValueError("calibration inputs must be finite")
    return (2.0 / X.shape[0]) * (X.T @ X)


def gptq_factor_ref(H, damp=DAMP):
    """Damped Hessian's inverse factor: U upper triangular with (H + lambda I)^-1 = U^T U.

    Dead columns (H_jj = 0) get H_jj = 1 first; lambda = damp * mean(diag H).
    """
    H = np.array(H, dtype=np.float64, copy=True)
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    H[np.diag_indices_from(H)] += damp * np.mean(np.diag(H))
    # Cholesky of the inverse, upper form: H^-1 = L L^T with L lower, so U = L^T.
    L = np.linalg.cholesky(np.linalg.inv(H))
    return L.T


def _round_half_away(t32):
    t = t32.astype(np.float64)
    return np.trunc(t + np.copysign(0.5, t))


def group_scale_ref(w_group):
    """RTN's scale of each row of a group of current weights: fl32(max |fl32(w)| / 7)."""
    a = np.abs(w_group.astype(np.float32)).max(axis=1).astype(np.float32)
    return (a / np.float32(7.0)).astype(np.float32)


def code_ref(w, d):
    """RTN's code decision for one column of current weights against the group's scales."""
    usable = d != 0
    dd = np.where(usable, d, np.float32(1.0)).astype(np.float32)
    t = (w.astype(np.float32) / dd).astype(np.float32)
    q = np.clip(_round_half_away(t), QMIN, QMAX)
    return np.where(usable, q, 0.0)


def gptq_quantize_ref(W, U, block=GROUP, scale_dtype="f32"):
    """Codes and scales for W [N, K] (fp32, finite) given the inverse factor U [K, K].

    Returns (q int8 [N, K], d [N, K/128]): the same arrays RTN returns -- float32
    scales, or uint16 bf16 bit patterns for scale_dtype "bf16".  `block` is the
    lazy-update width; the group scale is always taken every 128 columns (a
    block width that is a multiple of 128 changes only the rounding order of the
    corrections).
    """
    if scale_dtype not in ("f32", "bf16"):
        raise ValueError("scale_dtype must be 'f32' or 'bf16'")
    W = np.asarray(W)
    if W.dtype != np.float32 or W.ndim != 2:
        raise TypeError("W must be a 2-D float32 array")
    N, K = W.shape
    if K <= 0 or K % GROUP or block % GROUP:
        raise ValueError("K and the block width must be positive multiples of 128")
    if not np.isfinite(W).all():
        raise ValueError("weights must be finite")
    U = np.asarray(U, dtype=np.float64)
    Wk = W.astype(np.float64)
    q = np.zeros((N, K), dtype=np.int8)
    d = np.zeros((N, K // GROUP), dtype=np.float32)  # the scales the codes use
    for b0 in range(0, K, block):
        b1 = min(b0 + block, K)
        E = np.zeros((N, b1 - b0))
        for j in range(b0, b1):
            if j % GROUP == 0:
                dj = group_scale_ref(Wk[:, j:j + GROUP])
                if scale_dtype == "bf16":  # stored as bf16; used widened back to fp32
                    dj = (f32_to_bf16_bits(dj).astype(np.uint32) << np.uint32(16)).view(np.float32)
                d[:, j // GROUP] = dj
            dg = d[:, j // GROUP]
            qj = code_ref(Wk[:, j], dg)
            q[:, j] = qj.astype(np.int8)
            err = (Wk[:, j] - dg.astype(np.float64) * qj) / U[j, j]
            Wk[:, j + 1:b1] -= np.outer(err, U[j, j + 1:b1])
            E[:, j - b0] = err
        Wk[:, b1:] -= E @ U[b0:b1, b1:]
    if scale_dtype == "bf16":
        return q, (d.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return q, d


def gptq_ref(W, x_bits, damp=DAMP, scale_dtype="f32"):
    """The whole procedure: Hessian from calibration rows, factor, column loop."""
    return gptq_quantize_ref(W, gptq_factor_ref(gptq_hessian_ref(x_bits), damp), scale_dtype=scale_dtype)


def output_error_ref(W, q, d, x_bits):
    """Mean squared output error of (q, d) against W on the rows x: mean((x W_hat^T - x W^T)^2), fp64."""
    X = bf16_bits_to_f64(x_bits)
    G = W.shape[1] // GROUP
    d = np.asarray(d)
    if d.dtype == np.uint16:  # bf16 scales
        d = bf16_bits_to_f64(d)
    What = (np.asarray(d, dtype=np.float64)[:, :, None] * q.reshape(q.shape[0], G, GROUP)).reshape(q.shape)
    return float(np.mean((X @ (What - np.asarray(W, dtype=np.float64)).T) ** 2))
