"""Dequantize-times-activation linear layer (oracle, fp64).

Computes y = W_hat x for a batch of M activation rows, where W_hat = d * q is
the restored weight of the group-quantization equation (Qwen3.5-4B quantization
study, section 1; z = 0) and y = W x is that section's linear layer (W is
N x K: N outputs, K inputs).  Inputs stay BF16 (section 2 settings table).
Decode re-runs this layer at M = 1, and verifying K drafted tokens runs it at
M = K + 1 rows in one pass (27B quantization-and-drafter ladder, stage 2).

Everything is widened to fp64 first: d * q is exact in fp64 (a 24-bit
significand times an integer below 16), bf16 -> fp64 is exact, and the
product is an ordinary float64 matrix product.

Non-finite activations (the pages are silent): a NaN or infinity anywhere in
row m of x makes every output of that row NaN -- the row is poisoned, as a
non-finite weight group poisons the outputs that use it -- instead of the
mix of +-inf and NaN that IEEE arithmetic of the sum would give.
"""

import numpy as np

from .bf16 import bf16_bits_to_f64
from .rtn import GROUP


def dequantize_ref(q, d):
    """W_hat[n, k] = d[n, k // 128] * q[n, k] in float64, [N, K].

    d: float32 scales, or uint16 bf16 bit patterns (16-bit scales)."""
    q = np.asarray(q)
    d = np.asarray(d)
    N, K = q.shape
    if d.shape != (N, K // GROUP):
        raise ValueError("d must be [N, K/128]")
    d64 = bf16_bits_to_f64(d) if d.dtype == np.uint16 else d.astype(np.float64)
    return np.repeat(d64, GROUP, axis=1) * q.astype(np.float64)


def w4_linear_ref(x_bits, q, d):
    """y[m, n] = sum_k x[m, k] * W_hat[n, k].

    x_bits: uint16 [M, K] bf16 bit patterns; q: int8 [N, K]; d: float32 [N, K/128]
    (or uint16 bf16 bit patterns for 16-bit scales).
    Returns (y, absdot), both float64 [M, N]; absdot = sum_k |x[m,k] * W_hat[n,k]|
    is the scale the output tolerance is stated against (oracle/tolerance.py).
    Rows of x holding a NaN or an infinity give NaN in y and absdot.
    """
    x = bf16_bits_to_f64(x_bits)
    w_hat = dequantize_ref(q, d)
    if x.ndim != 2 or x.shape[1] != w_hat.shape[1]:
        raise ValueError("x must be [M, K]")
    poisoned = ~np.isfinite(x).all(axis=1)
    x = np.where(poisoned[:, None], 0.0, x)
    y = x @ w_hat.T
    absdot = np.abs(x) @ np.abs(w_hat).T
    y[poisoned, :] = np.nan
    absdot[poisoned, :] = np.nan
    return y, absdot
