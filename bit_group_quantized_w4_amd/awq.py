"""Exponent search of the channel scaling before RTN (the AWQ recipe of the
Qwen3.5-4B quantization study, section 2: candidate scales from input
statistics only, s_j proportional to (mean |x_j|)^alpha for alpha = k/19,
k = 0..19, compared by the output error on calibration inputs; no clipping
search).  Every step runs in the library's kernels, the reference output
W x of the unquantized layer included (w4_dense_linear_f32, fp32).  The host
only picks the smallest of the 20 errors (ties to the smaller exponent).
"""

import torch

from . import awq_scales, channel_absmean, dense_linear_f32, linear, quantize_rtn_scaled, scale_activations, sq_error

ALPHAS = tuple(k / 19 for k in range(20))


def search(W, x_cal, scale_dtype=torch.float32):
    """W: fp32 [N, K] weights and x_cal: bf16 [T, K] calibration rows, both on the GPU.

    Returns a dict with the chosen index `k` and exponent `alpha`, the channel
    scales `s` and their reciprocals `inv_s` (fp32 [K]), the quantized scaled
    weight `q`, `d` (native layout), and `errors`: the mean squared output
    error of every candidate (a list of 20 floats).
    """
    N, K = W.shape
    T = x_cal.shape[0]
    m = channel_absmean(x_cal)
    y_ref = dense_linear_f32(x_cal, W)  # W x of the unquantized layer, fp32
    errs = torch.empty(len(ALPHAS), dtype=torch.float64, device=W.device)
    x_s = torch.empty_like(x_cal)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=W.device)
    for i, alpha in enumerate(ALPHAS):
        s, inv = awq_scales(m, alpha)
        q, d = quantize_rtn_scaled(W, s, scale_dtype)
        scale_activations(x_cal, inv, out=x_s)
        linear(x_s, q, d, N, out=y)
        sq_error(y, y_ref, out=errs[i:i + 1])
    errors = (errs.cpu() / float(T * N)).tolist()
    k = min(range(len(errors)), key=lambda i: (errors[i], i))
    s, inv = awq_scales(m, ALPHAS[k])
    q, d = quantize_rtn_scaled(W, s, scale_dtype)
    return {"k": k, "alpha": ALPHAS[k], "s": s, "inv_s": inv, "q": q, "d": d, "errors": errors}
