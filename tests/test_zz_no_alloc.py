"""w4_chain_prepare_noalloc: the chained pass set up in the library's static
device scratch, for callers that cannot allocate device memory.

Through the C ABI: its passes equal, bit for bit, those of the same chain
prepared with a caller workspace (w4_chain_prepare), on two chains prepared
one after the other (the second smaller, so it runs on what the first left in
the scratch), with the error flag clear; a chain that does not fit the
scratch is refused with W4_ERR_SCRATCH.
"""

import ctypes

import pytest
import torch

import workloads
from tests.test_gpu_chain import _build_chain
from tests.test_gpu_parity import _say

pytestmark = pytest.mark.gpu


def _outputs(records):
    return [r[7].view(torch.int16).clone() for r in records]


def _run_both(w4, gpu, layers, hidden, nq, nkv, ffn, seed):
    stages, records, x0 = _build_chain(w4, gpu, layers=layers, hidden=hidden, nq=nq, nkv=nkv, ffn=ffn, seed=seed)
    ref = w4.chain_prepare(stages)
    ref.run()
    assert ref.error() == 0
    want = _outputs(records)
    for r in records:
        r[7].zero_()
    plan = w4.chain_prepare(stages, noalloc=True)
    assert plan.workspace is None
    assert plan.plan.workspace != ref.plan.workspace
    plan.run()
    assert plan.error() == 0, "a wait of the no-allocation pass timed out"
    got = _outputs(records)
    for (name, *_), a, b in zip(records, want, got):
        assert torch.equal(a, b), f"{name}: the no-allocation pass differs from the workspace pass"
    # a second pass with a new input agrees as well
    x0.copy_(workloads.random_activations(1, hidden, seed=seed + 100, device=gpu))
    plan.run()
    assert plan.error() == 0
    got = _outputs(records)
    ref.run()
    assert ref.error() == 0
    for (name, *_), a, b in zip(records, _outputs(records), got):
        assert torch.equal(a, b), f"{name}: second pass differs"
    return plan


def test_noalloc_matches_workspace_entry(w4, gpu):
    _say("no-allocation chain: 3 layers (hidden 1024), then 1 layer (hidden 512)")
    first = _run_both(w4, gpu, layers=3, hidden=1024, nq=1024, nkv=256, ffn=2816, seed=41)
    second = _run_both(w4, gpu, layers=1, hidden=512, nq=768, nkv=256, ffn=1408, seed=42)
    assert first.plan.workspace == second.plan.workspace  # one scratch per GPU
    assert second.plan.linears < first.plan.linears


def test_noalloc_refuses_a_chain_beyond_the_scratch(w4, gpu):
    _say("no-allocation chain: a chain longer than the scratch holds")
    lib = w4.library()
    K, N = 128, 16
    W = torch.from_numpy(workloads.random_weight(N, K, seed=43)).to(gpu)
    q, d = w4.quantize_rtn(W)
    x = workloads.random_activations(1, K, seed=43, device=gpu)
    n = 1023  # the scratch (65536 bytes) holds a header and 1023 table entries: 1022 linears and the end marker
    ys = torch.empty((n, 128), dtype=torch.bfloat16, device=gpu)  # one 256-byte row per output
    descs = (w4.ChainLinear * n)(*[w4.ChainLinear(x.data_ptr(), 1, K, q.data_ptr(), d.data_ptr(), N,
                                                  ys[i].data_ptr(), 0) for i in range(n)])
    plan = w4.ChainPlanC()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.w4_chain_workspace_bytes(n) > 65536
    assert lib.w4_chain_prepare_noalloc(descs, n, ctypes.byref(plan), stream) == w4.W4_ERR_SCRATCH
    assert b"W4_ERR_SCRATCH" in lib.w4_status_str(w4.W4_ERR_SCRATCH)
    # one linear fewer fits, and runs
    assert lib.w4_chain_workspace_bytes(n - 1) <= 65536
    assert lib.w4_chain_prepare_noalloc(descs, n - 1, ctypes.byref(plan), stream) == w4.W4_OK
    assert lib.w4_chain_run(ctypes.byref(plan), stream) == w4.W4_OK
    flag = ctypes.c_uint32(1)
    assert lib.w4_chain_error(ctypes.byref(plan), ctypes.byref(flag), stream) == w4.W4_OK
    assert flag.value == 0
    ref = w4.linear(x, q, d, N)
    torch.cuda.synchronize()
    assert torch.equal(ys[:n - 1, :N].view(torch.int16), ref.view(torch.int16).expand(n - 1, N))
