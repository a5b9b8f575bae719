"""Every output of the timed stack passes, checked.

The measured passes run every linear of a stack: the chained decode pass
(one w4_chain_run over all layers, each stage reading the previous stage's
output; the 70B-class pass at M = 1 is the headline) and the verification
pass with one launch per shared-input group (split workspace given).  These
tests build those passes exactly as bench.py does (its chain_stages and its
fused groups; the same weights, drawn on the GPU, and the same activations),
run them once, and check every output element of every linear of every layer
against the product of the codes and scales that linear used, evaluated with
plain torch operations in fp64:

* w_hat[n, k] = d[n, k / 128] * q[n, k] (exact in fp64), from w4_unpack;
* y_ref = x @ w_hat^T and absdot = |x| @ |w_hat|^T in fp64, x the bf16 input
  the linear actually read (for a chained stage: the previous stage's output);

to the accuracy convention of oracle.admissible, wherever the input lies in
the range where that bound is promised (every |x| at most 2^64; the weights
here are far inside theirs).  The chained pass feeds each stage the previous
stage's output with no normalization between layers, so its activations grow
by every linear's gain; on the 70B-class stack they leave that range after
about a dozen layers and overflow fp32 later.  Past the range the promise is
weaker and is what is checked there: no output is a wrong finite value (each
finite output is admissible; the others may be infinite or NaN).  The codes and scales
themselves are held to the group-quantization equation on every element by
test_gpu_stack_codes.py.  The fp64 evaluation is tied to the CPU oracle
(oracle.rtn_quantize_ref, then oracle.w4_linear_ref, on the same rows of W)
on 8 sampled rows of every linear.
"""

import numpy as np
import pytest
import torch

import bench
import oracle
import workloads
from tests.test_gpu_parity import _bits, _say, check_y

pytestmark = pytest.mark.gpu

GROUP = 128
TIE_ROWS = 8


def _quantized_stack(w4, gpu, name, rng):
    """Per layer: (matrix, q, d, sampled row indices, those rows of W in fp32 on the host)."""
    wl = workloads.WORKLOADS[name]
    layers = []
    for layer in range(wl.layers):
        mats = []
        for m in wl.matrices:
            W = workloads.weight(name, layer, m.name, gpu)
            q, d = w4.quantize_rtn(W)
            rows = np.sort(rng.choice(m.N, TIE_ROWS, replace=False))
            W_rows = W.index_select(0, torch.as_tensor(rows, device=gpu)).cpu().numpy()
            del W
            mats.append((m, q, d, rows, W_rows))
        layers.append(mats)
    return layers


def _fp64_reference(w4, x, q, d, N):
    """(y_ref, absdot) as fp64 [M, N] host arrays for bf16 x [M, K] on the device."""
    K = x.shape[1]
    qc, dc = w4.unpack(q, d, N, K)
    w_hat = qc.double() * dc.double().repeat_interleave(GROUP, dim=1)
    x64 = x.double()
    y_ref = (x64 @ w_hat.T).cpu().numpy()
    absdot = (x64.abs() @ w_hat.abs().T).cpu().numpy()
    return y_ref, absdot


X_RANGE = 2.0 ** 64  # largest |x| for which every output is promised within tolerance


def _check_linear(w4, what, x, q, d, N, y, rows, W_rows):
    """True if x was within the range (and every output was checked as such)."""
    y_ref, absdot = _fp64_reference(w4, x, q, d, N)
    xmax = x.float().abs().max().item()
    if not xmax <= X_RANGE:  # past the range (or non-finite): no wrong finite value
        bits = _bits(y)
        y_gpu = oracle.bf16_bits_to_f64(bits)
        fin = np.isfinite(y_gpu)
        with np.errstate(invalid="ignore"):
            ok = oracle.admissible(bits, y_ref, absdot, "bf16")
        assert np.all(ok[fin]), f"{what} (|x| up to {xmax:.3g}): {int(np.sum(~ok[fin]))} wrong finite outputs"
        return False
    check_y(y, y_ref, absdot, what)
    # The fp64 evaluation against the oracle on the sampled rows: both sum the
    # same K exact products in some order, so they differ by at most twice
    # the worst-case summation error, K * 2^-53 * absdot each.
    q_o, d_o = oracle.rtn_quantize_ref(W_rows)
    y_o, absdot_o = oracle.w4_linear_ref(_bits(x), q_o, d_o)
    bound = 2.0 * x.shape[1] * 2.0 ** -53 * absdot_o
    assert np.all(np.abs(y_ref[:, rows] - y_o) <= bound), f"{what}: fp64 evaluation differs from the oracle"
    assert np.all(np.abs(absdot[:, rows] - absdot_o) <= bound), f"{what}: absdot differs from the oracle"
    return True


@pytest.mark.parametrize("name,M", [("stack_70b", 1), ("stack_27b", 1), ("stack_4b", 1), ("stack_27b", 8)])
def test_chained_pass_every_output(w4, gpu, name, M):
    """The chained pass (dot2 items at M = 1, MFMA items at M = 8)."""
    _say(f"chained pass {name} M={M}: every output of every linear")
    wl = workloads.WORKLOADS[name]
    layers = _quantized_stack(w4, gpu, name, np.random.default_rng(17 + M))
    xs = {m.K: workloads.activations(name, 0, m.name, M, gpu) for m in wl.matrices}
    stages, kinds = bench.chain_stages(torch, wl, [[(m, q, d) for m, q, d, _, _ in mats] for mats in layers], xs, M)
    plan = w4.chain_prepare(stages)
    plan.run()
    torch.cuda.synchronize()
    assert plan.error() == 0, "a chain wait timed out"
    samples = [(r, Wr) for mats in layers for _, _, _, r, Wr in mats]
    checked, in_range = 0, 0
    for si, (st, kind) in enumerate(zip(stages, kinds)):
        for j, (x, q, d, N, y) in enumerate(st):
            rows, W_rows = samples[checked]
            in_range += _check_linear(w4, f"{name} M={M} stage {si} ({kind}) linear {j}", x, q, d, N, y, rows, W_rows)
            checked += 1
    assert checked == len(wl.matrices) * wl.layers
    print(f"[case] {name} M={M}: {checked} linears, {in_range} with every |x| <= 2^64 "
          f"(checked against the bound), {checked - in_range} past that range", flush=True)
    # the first layers always start from the N(0, 1) activations
    assert in_range >= 7 * len(wl.matrices)
    del plan, stages, layers
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,M", [("stack_70b", 8), ("stack_70b", 16)])
def test_verification_pass_every_output(w4, gpu, name, M):
    """One launch per shared-input group with the split workspace, as the
    verification widths are timed; every layer."""
    _say(f"verification pass {name} M={M}: every output of every linear")
    wl = workloads.WORKLOADS[name]
    layers = _quantized_stack(w4, gpu, name, np.random.default_rng(29 + M))
    xs = {m.K: workloads.activations(name, 0, m.name, M, gpu) for m in wl.matrices}
    ws = w4.SplitWorkspace(gpu)
    groups = bench._shared_input_groups(wl)
    for layer, mats in enumerate(layers):
        ys = [torch.empty((M, m.N), dtype=torch.bfloat16, device=gpu) for m, *_ in mats]
        for gi in groups:
            if len(gi) == 1:
                m, q, d, _, _ = mats[gi[0]]
                w4.linear(xs[m.K], q, d, m.N, out=ys[gi[0]], workspace=ws)
            else:
                w4.linear_batched([(xs[mats[i][0].K], mats[i][1], mats[i][2], mats[i][0].N, ys[i]) for i in gi],
                                  workspace=ws)
        torch.cuda.synchronize()
        assert ws.error() == 0, "a split wait timed out"
        for i, (m, q, d, rows, W_rows) in enumerate(mats):
            assert _check_linear(w4, f"{name} M={M} layer {layer} {m.name}", xs[m.K], q, d, m.N, ys[i], rows, W_rows)
    del layers
    torch.cuda.empty_cache()
