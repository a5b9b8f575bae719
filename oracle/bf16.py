"""Decoding of bfloat16 bit patterns (oracle side).

BF16 is the activation precision of the method (Qwen3.5-4B quantization study,
section 2 settings table: 4-bit weights, BF16 inputs).  A bf16 value is the top
16 bits of an IEEE binary32, so widening it is exact.
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
