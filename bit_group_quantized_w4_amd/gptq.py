"""GPTQ quantizer (the study's section 2: GPTQ row of the methods table and
its settings -- damping 0.01 of the mean Hessian diagonal, 128-column blocks,
no reordering, RTN's storage; update rule of the published GPTQ algorithm).

Every step runs in the library's kernels: the Hessian X^T X in fp64
(w4_gptq_hessian), its damping (w4_gptq_damp), the factor U of the damped
Hessian's inverse, H^-1 = U^T U, by a blocked fp64 Cholesky factorization and
triangular inverse (w4_gptq_inverse_factor), the column loop of every block
with its code decisions and in-block corrections (w4_gptq_block), the product
correcting the columns after each block (w4_gptq_update), and the packing
into the native layout (w4_pack).  PyTorch only provides the buffers and the
stream.
"""

import torch

from . import gptq_block, gptq_damp, gptq_hessian, gptq_inverse_factor, gptq_update, pack

DAMP = 0.01
BLOCK = 128


def hessian(x_cal):
    """H = (2/T) X^T X, fp64 [K, K], from bf16 calibration rows [T, K]."""
    return gptq_hessian(x_cal)


def inverse_factor(H):
    """U upper triangular (fp32) with H^-1 = U^T U (H damped; not modified)."""
    return gptq_inverse_factor(H)


def quantize(W, x_cal, damp=DAMP, timings=None, scale_dtype=torch.float32):
    """GPTQ of W (fp32 [N, K], K a multiple of 128, finite) with calibration rows x_cal
    (bf16 [T, K]).  Returns (q, d) in the native layout, as quantize_rtn does; with
    scale_dtype=torch.bfloat16 the scales are 16-bit (the codes use the stored values).

    With a dict `timings`, the milliseconds of each phase (GPU events on the
    current stream) are stored in it: "hessian", "factor", "columns" (the block
    loops with their corrections) and "pack"."""
    if W.dim() != 2 or W.dtype != torch.float32 or not W.is_cuda:
        raise TypeError("W must be a 2-D float32 tensor on the GPU")
    if x_cal.dim() != 2 or x_cal.dtype != torch.bfloat16 or x_cal.device != W.device:
        raise TypeError("x_cal must be a 2-D bfloat16 tensor on W's device")
    N, K = W.shape
    if K == 0 or K % BLOCK:
        raise ValueError("K must be a positive multiple of 128")
    if x_cal.shape[1] != K or x_cal.shape[0] < 1:
        raise ValueError("x_cal must have at least one row of K inputs")
    if not (damp >= 0.0 and damp < float("inf")):
        raise ValueError("damp must be finite and >= 0")
    if scale_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("scale_dtype must be torch.float32 or torch.bfloat16")
    marks = []

    def mark():
        if timings is not None:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            marks.append(e)

    mark()
    H = hessian(x_cal)
    gptq_damp(H, damp)
    mark()
    U = inverse_factor(H)
    del H
    mark()
    Wk = W.clone()
    q_canon = torch.empty((N, K), dtype=torch.int8, device=W.device)
    d_canon = torch.empty((N, K // BLOCK), dtype=scale_dtype, device=W.device)
    err = torch.empty((BLOCK, N), dtype=torch.float32, device=W.device)
    for b0 in range(0, K, BLOCK):
        gptq_block(Wk, U, b0, q_canon, d_canon, err)
        gptq_update(Wk, U, b0, err)
    mark()
    q, d = pack(q_canon, d_canon)
    mark()
    if timings is not None:
        marks[-1].synchronize()
        for name, a, b in zip(("hessian", "factor", "columns", "pack"), marks, marks[1:]):
            timings[name] = a.elapsed_time(b)
    return q, d
