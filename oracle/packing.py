"""Canonical byte order for 4-bit codes (oracle side).

A 4-bit slot holds one of 16 codes (Qwen3.5-4B quantization study, section 1
symbol table), so two codes share a byte.  The canonical order used to compare
codes bit for bit is row-major [N][K/2]: byte k/2 of row n holds code k in its
low nibble and code k+1 in its high nibble, each stored offset-binary as
u = q + 8 (0..15).  The offset is a storage choice only; the value is still
w_hat = d * q with zero point 0.
"""

import numpy as np


def pack_canonical(q):
    """int8 codes [N, K] in [-8, 7] -> uint8 [N, K/2]."""
    q = np.asarray(q)
    if q.ndim != 2 or q.shape[1] % 2:
        raise ValueError("q must be [N, K] with K even")
    if q.size and (q.min() < -8 or q.max() > 7):
        raise ValueError("codes must lie in [-8, 7]")
    u = (q.astype(np.int16) + 8).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_canonical(b):
    """uint8 [N, K/2] -> int8 codes [N, K]."""
    b = np.asarray(b, dtype=np.uint8)
    N, H = b.shape
    q = np.empty((N, 2 * H), dtype=np.int8)
    q[:, 0::2] = (b & 0x0F).astype(np.int16) - 8
    q[:, 1::2] = (b >> 4).astype(np.int16) - 8
    return q
