"""Split launches (w4_linear_batched_split*) on an MI355X, through the C ABI,
against the CPU oracle on the same seeded inputs.

The MFMA kernel divides each row panel's inputs among S blocks; S - 1 of them
publish fp32 partial sums in the workspace and the panel's last block adds
them in slice order.  Checked here:

* every output is a correct result for the oracle's exact value (the
  accuracy convention of oracle/tolerance.py), for S forced to 2, 3, 4 and 8
  and for the automatic choice, on several split-K configurations, ragged N
  and K, M from 1 to 16 (and 17: two slabs of x), bf16 and fp32 outputs, fp32
  and bf16 scales, single and batched launches;
* results are reproducible: the same call twice gives the same bits;
* the workspace is left initialised (error word zero, every slot unwritten),
  and its error word stays zero;
* non-finite activations still poison exactly their rows, including the bf16
  pattern 0xFFFF, whose widening is the unwritten-slot pattern's upper half;
* a workspace that was never initialised is detected on the device: the split
  outputs are NaN, nothing waits, and the error word has bit 1 set.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.test_gpu_parity import _bits, _say, check_y

pytestmark = pytest.mark.gpu

SPLIT_CFGS = ["2,4", "1,4", "4,4", "2,2", "1,8", "4,1", "2,8s", "2,4s"]
SHAPES = [(700, 2048), (37, 4224), (260, 9216)]


@pytest.fixture(scope="module")
def ws(w4, gpu):
    return w4.SplitWorkspace(gpu)


def _quantized(w4, gpu, N, K, seed, scale_dtype="f32"):
    W = workloads.random_weight(N, K, seed=seed)
    sd = torch.bfloat16 if scale_dtype == "bf16" else torch.float32
    q, d = w4.quantize_rtn(torch.from_numpy(W).to(gpu), scale_dtype=sd)
    q_ref, d_ref = oracle.rtn_quantize_ref(W, scale_dtype)
    return q, d, q_ref, d_ref


def check_workspace_clean(ws):
    """Error word zero and every slot back to the unwritten pattern."""
    b = ws.buffer.cpu().numpy()
    words = b.view(np.uint32)
    assert words[0] == 0, "error word set"
    assert np.all(words[64:] == 0xFFFFFFFF), f"{int(np.sum(words[64:] != 0xFFFFFFFF))} slot words left written"


@pytest.mark.parametrize("S", ["2", "3", "4", "8", None])
@pytest.mark.parametrize("cfg", SPLIT_CFGS)
def test_split_matches_oracle(w4, gpu, ws, cfg, S, monkeypatch):
    monkeypatch.setenv("W4_MFMA_CFG", cfg)
    if S:
        monkeypatch.setenv("W4_MFMA_SPLIT", S)
    for i, (N, K) in enumerate(SHAPES):
        q, d, q_ref, d_ref = _quantized(w4, gpu, N, K, seed=300 + i)
        for M in (1, 5, 8, 16, 17):
            _say(f"split cfg={cfg} S={S or 'auto'} {N}x{K} M={M}")
            x = workloads.random_activations(M, K, seed=M + 7 * i, device=gpu)
            y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
            yb = w4.linear(x, q, d, N, path="mfma", workspace=ws)
            yb2 = w4.linear(x, q, d, N, path="mfma", workspace=ws)
            yf = w4.linear(x, q, d, N, path="mfma", out_dtype=torch.float32, workspace=ws)
            check_y(yb, y_ref, absdot, f"bf16 {N}x{K} M={M}")
            check_y(yf, y_ref, absdot, f"fp32 {N}x{K} M={M}")
            assert torch.equal(yb.view(torch.int16), yb2.view(torch.int16)), "not reproducible"
            # bf16 outputs are the rounding of the fp32 outputs of the same split
            assert np.array_equal(_bits(yb), oracle.f32_to_bf16_bits(yf.cpu().numpy()))
    check_workspace_clean(ws)


@pytest.mark.parametrize("scale_dtype", ["f32", "bf16"])
def test_split_batched_decoder_layer(w4, gpu, ws, scale_dtype, monkeypatch):
    """q|k|v and gate|up of a 4B-class layer as split batches at M = 8 and 13."""
    monkeypatch.setenv("W4_MFMA_CFG", "2,4")
    monkeypatch.setenv("W4_MFMA_SPLIT", "3")
    wl = workloads.WORKLOADS["stack_4b"]
    mats = {m.name: m for m in wl.matrices}
    for group in (["q", "k", "v"], ["gate", "up"], ["down"]):
        qs = [_quantized(w4, gpu, mats[n].N, mats[n].K, seed=400 + j, scale_dtype=scale_dtype)
              for j, n in enumerate(group)]
        K = mats[group[0]].K
        for M in (8, 13):
            _say(f"split batched {'|'.join(group)} M={M} scales={scale_dtype}")
            x = workloads.activations("stack_4b", 0, group[0], M, gpu)
            ys = [torch.empty((M, mats[n].N), dtype=torch.bfloat16, device=gpu) for n in group]
            w4.linear_batched([(x, q, d, mats[n].N, y) for n, (q, d, _, _), y in zip(group, qs, ys)],
                              path="mfma", workspace=ws)
            for n, (_, _, q_ref, d_ref), y in zip(group, qs, ys):
                y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
                check_y(y, y_ref, absdot, f"{n} M={M}")
    check_workspace_clean(ws)


def test_split_full_size_down_projection(w4, gpu, ws):
    """The 70B-class down projection (8192 x 28672) at M = 16 with the automatic
    configuration and split, on sampled output columns."""
    N, K, M = 8192, 28672, 16
    _say(f"split full-size down {N}x{K} M={M}")
    W = workloads.weight("stack_70b", 0, "down", gpu)
    q, d = w4.quantize_rtn(W)
    x = workloads.activations("stack_70b", 0, "down", M, gpu)
    y = w4.linear(x, q, d, N, path="mfma", workspace=ws)
    cols = np.random.default_rng(5).choice(N, 96, replace=False)
    Wc = W[torch.from_numpy(cols).to(gpu)].cpu().numpy()
    del W
    q_ref, d_ref = oracle.rtn_quantize_ref(Wc)
    y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
    check_y(y[:, torch.from_numpy(cols).to(gpu)].contiguous(), y_ref, absdot, "down sampled columns")
    assert ws.error() == 0
    check_workspace_clean(ws)


@pytest.mark.parametrize("K", [4096, 2688])
def test_split_nonfinite_rows(w4, gpu, ws, K, monkeypatch):
    """(K = 2688: the last scale quad is padded; the NaN in row 1 at column 5
    must not reach row 0 through the padding's x.)"""
    monkeypatch.setenv("W4_MFMA_CFG", "2,4")
    monkeypatch.setenv("W4_MFMA_SPLIT", "4")
    N, M = 300, 16
    q, d, q_ref, d_ref = _quantized(w4, gpu, N, K, seed=77)
    x = workloads.random_activations(M, K, seed=9, device=gpu)
    xb = x.view(torch.int16)
    xb[1, 5] = -1            # bf16 0xFFFF: a NaN with every payload bit set
    xb[4, K - 1] = 0x7F80    # +inf
    xb[9, 2000] = -128       # 0xFF80: -inf
    _say(f"split non-finite rows K={K}")
    y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
    assert np.isnan(y_ref[[1, 4, 9]]).all()
    for od in (torch.bfloat16, torch.float32):
        y = w4.linear(x, q, d, N, path="mfma", out_dtype=od, workspace=ws)
        check_y(y, y_ref, absdot, f"non-finite rows {od}")
    assert ws.error() == 0
    check_workspace_clean(ws)


def test_split_workspace_reuse_after_smaller_call(w4, gpu, ws, monkeypatch):
    """A large split call, then a smaller one on the same workspace, then the
    large one again: every result correct and identical to the first."""
    monkeypatch.setenv("W4_MFMA_CFG", "1,4")
    monkeypatch.setenv("W4_MFMA_SPLIT", "8")
    big = _quantized(w4, gpu, 1024, 8192, seed=11)
    small = _quantized(w4, gpu, 48, 1024, seed=12)
    xb = workloads.random_activations(16, 8192, seed=13, device=gpu)
    xs = workloads.random_activations(3, 1024, seed=14, device=gpu)
    _say("split workspace reuse")
    y1 = w4.linear(xb, big[0], big[1], 1024, path="mfma", workspace=ws)
    y2 = w4.linear(xs, small[0], small[1], 48, path="mfma", workspace=ws)
    y3 = w4.linear(xb, big[0], big[1], 1024, path="mfma", workspace=ws)
    for y, x, (_, _, q_ref, d_ref) in ((y1, xb, big), (y2, xs, small)):
        y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
        check_y(y, y_ref, absdot, "reuse")
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
    check_workspace_clean(ws)


def test_split_uninitialised_workspace(w4, gpu, monkeypatch):
    monkeypatch.setenv("W4_MFMA_CFG", "2,4")
    monkeypatch.setenv("W4_MFMA_SPLIT", "3")
    N, K, M = 300, 4096, 8
    q, d, q_ref, d_ref = _quantized(w4, gpu, N, K, seed=21)
    x = workloads.random_activations(M, K, seed=22, device=gpu)
    fresh = w4.SplitWorkspace(gpu)
    fresh.buffer.zero_()  # as if allocated and never initialised
    _say("split with an uninitialised workspace")
    y = w4.linear(x, q, d, N, path="mfma", workspace=fresh)
    assert torch.isnan(y.float()).all(), "outputs of an uninitialised workspace must be NaN"
    assert fresh.error() == 2
    fresh.init()
    y = w4.linear(x, q, d, N, path="mfma", workspace=fresh)
    y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
    check_y(y, y_ref, absdot, "after initialisation")
    assert fresh.error() == 0
    check_workspace_clean(fresh)
