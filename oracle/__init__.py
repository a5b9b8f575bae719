"""CPU oracle for group-wise symmetric INT4 (RTN) quantization and the W4A16 linear.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code, tables or helpers with the HIP
library under ``bit_group_quantized_w4_amd/``; the only thing both sides see is
the seeded synthetic input from ``workloads/``.

What it computes (sources are the public pages this project is built from):

* ``rtn_quantize_ref`` -- the group quantizer of the Qwen3.5-4B quantization
  study (parksieon.github.io/qwen35-4b-quantization-study), section 1 "what was
  compressed": the equation q = clip(round(w/d) + z, qmin, qmax), w_hat = d(q - z)
  with its symbol table, groups of 128 consecutive inputs along each row, and
  section 2's settings table (RTN, symmetric, min/max range, group 128, no
  clipping search).  Done in fp32, as the kernel does; optionally with the
  scale stored as bf16 (16-bit scales) and the codes taken against it.
* ``w4_linear_ref`` -- y = W_hat x from the same section 1 (the 2560x9216 FFN
  example) with 4-bit weights and BF16 inputs (section 2 settings table), in
  fp64.
* ``admissible`` -- when an output counts as correct: within 2e-3 of
  sum |w_hat x| (plus 1e-6) of the exact value for fp32 outputs, and the
  nearest-even bf16 of such a value for bf16 outputs.
* ``pack_canonical`` / ``unpack_canonical`` -- the canonical two-codes-per-byte
  byte order used to compare codes bit for bit.
* ``awq_search_ref`` and its steps -- activation-aware channel scaling before
  RTN (study, section 2: the AWQ row of the methods table, the 20-exponent
  scale search of the settings table, and the channel-scaling and
  output-error equations).
* ``gptq_ref`` and its steps -- GPTQ's column-by-column quantization with
  error feedback (study, section 2: the GPTQ row, damping 0.01, 128-column
  blocks, no reordering; the update rule of the published GPTQ algorithm).

Every function here is pinned by ``tests/test_oracle.py`` against exact
rational arithmetic, brute force on small inputs, closed forms and hand-derived
fixtures in ``tests/golden/``; none is "parity unpinned".
"""

from .awq import (ALPHAS, awq_output_error_ref, awq_search_ref, candidate_scales_ref, channel_absmean_ref,
                  quantize_scaled_ref, scale_activations_ref)
from .bf16 import bf16_bits_to_f64, f32_to_bf16_bits
from .gptq import gptq_factor_ref, gptq_hessian_ref, gptq_quantize_ref, gptq_ref, output_error_ref
from .linear import dequantize_ref, w4_linear_ref
from .packing import pack_canonical, unpack_canonical
from .rtn import GROUP, NAN_BITS, QMAX, QMIN, rtn_quantize_ref
from .tolerance import ABS_TOL, REL_TOL, admissible, rounding_interval, worst_ratio

__all__ = [
    "ABS_TOL",
    "ALPHAS",
    "GROUP",
    "NAN_BITS",
    "QMAX",
    "QMIN",
    "REL_TOL",
    "admissible",
    "awq_output_error_ref",
    "awq_search_ref",
    "candidate_scales_ref",
    "channel_absmean_ref",
    "quantize_scaled_ref",
    "scale_activations_ref",
    "bf16_bits_to_f64",
    "dequantize_ref",
    "f32_to_bf16_bits",
    "gptq_factor_ref",
    "gptq_hessian_ref",
    "gptq_quantize_ref",
    "gptq_ref",
    "output_error_ref",
    "pack_canonical",
    "rounding_interval",
    "rtn_quantize_ref",
    "unpack_canonical",
    "w4_linear_ref",
    "worst_ratio",
]
