"""GPTQ quantizer (the study's section 2: GPTQ row of the methods table and
its settings -- damping 0.01 of the mean Hessian diagonal, 128-column blocks,
no reordering, RTN's storage; update rule of the published GPTQ algorithm).

The method-specific steps run in the library's kernels: damping the Hessian
(w4_gptq_damp), the column loop of every block with its code decisions and
in-block corrections (w4_gptq_block) and the packing into the native layout
(w4_pack).  Three plain dense linear-algebra steps use the GPU libraries
PyTorch links: the Hessian product X^T X and the factorization of the damped
Hessian's inverse (one Cholesky factorization and one triangular inverse),
both in fp64 -- a strongly anisotropic Hessian (outlier input channels) loses
too much in an fp32 factorization -- and, in fp32, the product that corrects
the columns after each block.
"""

import torch

from . import gptq_block, gptq_damp, pack

DAMP = 0.01
BLOCK = 128


def hessian(x_cal):
    """H = (2/T) X^T X, fp64 [K, K], from bf16 calibration rows [T, K]."""
    X = x_cal.double()
    return (X.t() @ X).mul_(2.0 / X.shape[0])


def inverse_factor(H):
    """U upper triangular with H^-1 = U^T U.

    With J the index reversal, J H J = L L^T (L lower) gives H = V V^T for the
    upper triangular V = J L J, so H^-1 = (V^-1)^T V^-1 and U = V^-1 = J L^-1 J."""
    L = torch.linalg.cholesky(torch.flip(H, [0, 1]))
    eye = torch.eye(H.shape[0], dtype=H.dtype, device=H.device)
    return torch.flip(torch.linalg.solve_triangular(L, eye, upper=False), [0, 1]).contiguous()


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
    U = inverse_factor(H).float()
    del H
    mark()
    Wk = W.clone()
    q_canon = torch.empty((N, K), dtype=torch.int8, device=W.device)
    if scale_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("scale_dtype must be torch.float32 or torch.bfloat16")
    d_canon = torch.empty((N, K // BLOCK), dtype=scale_dtype, device=W.device)
    err = torch.empty((BLOCK, N), dtype=torch.float32, device=W.device)
    for b0 in range(0, K, BLOCK):
        gptq_block(Wk, U, b0, q_canon, d_canon, err)
        b1 = b0 + BLOCK
        if b1 < K:
            Wk[:, b1:].addmm_(err.t(), U[b0:b1, b1:], alpha=-1.0)
    mark()
    q, d = pack(q_canon, d_canon)
    mark()
    if timings is not None:
        marks[-1].synchronize()
        for name, a, b in zip(("hessian", "factor", "columns", "pack"), marks, marks[1:]):
            timings[name] = a.elapsed_time(b)
    return q, d
