"""Every code and scale of every layer of the 4B-, 27B- and 70B-class stacks.

The HIP quantizer (w4_quantize_rtn, and w4_quantize_rtn_s16 for 16-bit scales)
runs on every matrix of every layer, the weights drawn on the GPU exactly as
bench.py draws them.  Its codes and scales, unpacked to canonical order
(w4_unpack), must equal the group-quantization equation (Qwen3.5-4B
quantization study, section 1; the reading of the oracle's header) evaluated
on the same weights with plain torch operations:

* a = the group's largest magnitude (exact);
* d = fl32(a / 7), the divide taken in fp64 and rounded to fp32 -- fp64 has
  more than twice fp32's precision plus two bits, so this is the correctly
  rounded fp32 quotient whatever torch's fp32 divide does; with 16-bit scales
  the stored scale is bf16(d) (nearest even) and the codes use its value;
* q = clamp(round half away from zero of fl32(w / d), -8, 7), the rounding
  taken in fp64, where adding 1/2 to an fp32 quotient is exact.

That evaluation is tied to the CPU oracle (oracle.rtn_quantize_ref) on 32
sampled rows of every matrix of every layer.  The sampled tests of
test_gpu_parity.py check the HIP quantizer against the oracle directly; this
file closes the rest of every stack.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.test_gpu_parity import _say

pytestmark = pytest.mark.gpu

GROUP = 128


def rtn_reference(W, scale_dtype):
    """(codes int8 [N, K], scale bit patterns [N, K/128]) of the equation above."""
    N, K = W.shape
    Wg = W.view(N, K // GROUP, GROUP)
    a = Wg.abs().amax(dim=2)
    d = (a.double() / 7.0).float()
    if scale_dtype == torch.bfloat16:
        d16 = d.to(torch.bfloat16)
        d_used, d_bits = d16.float(), d16.view(torch.int16)
    else:
        d_used, d_bits = d, d.view(torch.int32)
    t = (Wg.double() / d_used.double()[:, :, None]).float().double()
    q = torch.trunc(t + torch.copysign(torch.full_like(t, 0.5), t)).clamp_(-8, 7)
    return q.to(torch.int8).view(N, K), d_bits


@pytest.mark.parametrize("workload,scale_dtype", [("stack_4b", torch.float32), ("stack_27b", torch.float32),
                                                  ("stack_70b", torch.float32), ("stack_27b", torch.bfloat16)])
def test_stack_codes_every_layer(w4, gpu, workload, scale_dtype):
    wl = workloads.WORKLOADS[workload]
    sd_name = "bf16" if scale_dtype == torch.bfloat16 else "f32"
    checked = 0
    for layer in range(wl.layers):
        if layer % 8 == 0:
            _say(f"stack codes {workload} ({sd_name} scales) layers {layer}..{min(layer + 7, wl.layers - 1)}")
        for m in wl.matrices:
            W = workloads.weight(workload, layer, m.name, gpu)
            q, d = w4.quantize_rtn(W, scale_dtype=scale_dtype)
            qc, dc = w4.unpack(q, d, m.N, m.K)
            q_ref, d_ref = rtn_reference(W, scale_dtype)
            bits = dc.view(torch.int16 if scale_dtype == torch.bfloat16 else torch.int32)
            assert torch.equal(bits, d_ref), f"{workload} layer {layer} {m.name}: scales differ"
            assert torch.equal(qc, q_ref), f"{workload} layer {layer} {m.name}: codes differ"
            rows = np.sort(np.random.default_rng(1000 * layer + m.N).choice(m.N, 32, replace=False))
            ridx = torch.as_tensor(rows, device=gpu)
            qo, do = oracle.rtn_quantize_ref(W.index_select(0, ridx).cpu().numpy(), sd_name)
            assert np.array_equal(q_ref.index_select(0, ridx).cpu().numpy(), qo), \
                f"{workload} layer {layer} {m.name}: reference codes differ from the oracle"
            want = do.view(np.int16) if sd_name == "bf16" else do.view(np.int32)
            assert np.array_equal(d_ref.index_select(0, ridx).cpu().numpy(), want), \
                f"{workload} layer {layer} {m.name}: reference scales differ from the oracle"
            checked += m.N * m.K
            del W, q, d, qc, dc, q_ref, d_ref
    torch.cuda.empty_cache()
    assert checked == workloads.stack_weights(workload)
