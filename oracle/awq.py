"""Activation-aware channel scaling before RTN (AWQ recipe of the study; oracle).

Qwen3.5-4B quantization study, section 2 ("what each method fixed"):

* AWQ keeps RTN's storage (symmetric INT4, group 128) and rescales input
  channels before quantizing: the weight column j is multiplied by s_j and the
  input x_j divided by it, so that W'x' = Wx with W'_ij = W_ij s_j and
  x'_j = x_j / s_j (the section's channel-scaling equation);
* the candidate scales come from input statistics only, s_j proportional to
  (mean |x_j|)^alpha with alpha = k/19, k = 0..19 (20 exponents in [0, 1]);
* the candidates are compared by the output error on calibration inputs,
  Delta y = (W_hat - W) x (the section's output-error equation), with no
  separate clipping search; s_j is not restricted to powers of two and is
  distinct from the group scale d.

Readings where the pages are silent:

* "proportional to": the constant is fixed by giving the scales a geometric
  mean of 1 (channels with mean |x_j| = 0 are treated as 1e-30);
* the scales are stored as fp32 (s32 = fl32(s)) together with their fp32
  reciprocals inv_s32 = fl32(1 / s32); the weight is scaled in fp32,
  W' = fl32(W * s32), then quantized by RTN (optionally with 16-bit scales);
* the scaled input is what the linear consumes in bf16:
  x' = bf16_rne(fl32(x * inv_s32));
* "output error": the mean over calibration rows and outputs of
  (y' - y)^2, y' = W_hat' x' (the quantized, scaled layer) and y = W x, both in
  fp64; the smallest error wins, ties to the smaller alpha.
"""

import numpy as np

from .bf16 import bf16_bits_to_f64, f32_to_bf16_bits
from .linear import w4_linear_ref
from .rtn import rtn_quantize_ref

ALPHAS = tuple(k / 19 for k in range(20))


def channel_absmean_ref(x_bits):
    """mean_t |x[t, j]| per input channel, fp64, from bf16 calibration rows [T, K]."""
    return np.abs(bf16_bits_to_f64(x_bits)).mean(axis=0)


def candidate_scales_ref(m, alpha):
    """Channel scales for one exponent: (s32, inv_s32), fp32 [K].

    s_j = p_j / exp(mean_i log p_i) with p_j = max(m_j, 1e-30)^alpha (fp64),
    then s32 = fl32(s) and inv_s32 = fl32(1 / s32)."""
    p = np.power(np.maximum(np.asarray(m, dtype=np.float64), 1e-30), float(alpha))
    s = p / np.exp(np.mean(np.log(p)))
    s32 = s.astype(np.float32)
    inv32 = (1.0 / s32.astype(np.float64)).astype(np.float32)
    return s32, inv32


def quantize_scaled_ref(W, s32, scale_dtype="f32"):
    """RTN of W' = fl32(W * s32) (columns scaled): (q, d) as rtn_quantize_ref."""
    Ws = (np.asarray(W, dtype=np.float32) * np.asarray(s32, dtype=np.float32)[None, :]).astype(np.float32)
    return rtn_quantize_ref(Ws, scale_dtype)


def scale_activations_ref(x_bits, inv_s32):
    """x' = bf16_rne(fl32(x * inv_s32)) as uint16 bf16 bit patterns [M, K]."""
    x32 = ((np.asarray(x_bits, dtype=np.uint16).astype(np.uint32)) << np.uint32(16)).view(np.float32)
    return f32_to_bf16_bits((x32 * np.asarray(inv_s32, dtype=np.float32)[None, :]).astype(np.float32))


def awq_output_error_ref(W, x_bits, s32, inv_s32, scale_dtype="f32"):
    """Mean squared output error of the scaled, quantized layer on calibration rows."""
    q, d = quantize_scaled_ref(W, s32, scale_dtype)
    y_q, _ = w4_linear_ref(scale_activations_ref(x_bits, inv_s32), q, d)
    y = bf16_bits_to_f64(x_bits) @ np.asarray(W, dtype=np.float64).T
    return float(np.mean((y_q - y) ** 2))


def awq_search_ref(W, x_bits, scale_dtype="f32"):
    """The exponent search: returns (k_best, s32, inv_s32, errors[20])."""
    m = channel_absmean_ref(x_bits)
    errors = []
    for alpha in ALPHAS:
        s32, inv32 = candidate_scales_ref(m, alpha)
        errors.append(awq_output_error_ref(W, x_bits, s32, inv32, scale_dtype))
    errors = np.asarray(errors)
    k = int(np.argmin(errors))  # first minimum: ties go to the smaller alpha
    s32, inv32 = candidate_scales_ref(m, ALPHAS[k])
    return k, s32, inv32, errors
