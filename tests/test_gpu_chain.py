"""Chained pass (w4_chain_prepare / w4_chain_run) on an MI355X.

A chain runs the linears of several decoder layers in stages, in one launch:
q|k|v read the layer input, o reads q's output, gate|up read o's output, down
reads gate's output, and the next layer reads down's output.  Every linear has
the same M: 1 (decode; dot2 items) or 2..16 (verification of drafted tokens;
MFMA items).  Each output must be (a) bitwise equal to one w4_linear_batched
call per stage with the chain's kernel (dot2 at M = 1, MFMA unsplit above) in
the chain's configuration, run on the very inputs the chain saw, and (b)
correct against the fp64 oracle on those inputs (oracle.admissible: the bf16
rounding of a value within 2e-3 * sum|w_hat x| + 1e-6).
Repeated passes, eager and graph-replayed, each with a new layer-0 input,
check that no pass reads a stale input and that the completion counters
return to zero.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.test_gpu_parity import _bits, _say, check_y

pytestmark = pytest.mark.gpu

CHAIN_CFGS = ["1,4", "1,8", "2,4", "2,2", "1,2", "4,4"]
CHAIN_MFMA_CFGS = ["2,4", "4,4", "1,4", "2,2"]


def _build_chain(w4, gpu, layers, hidden, nq, nkv, ffn, seed=0, side=True, same_sign=False, M=1):
    """Stages of `layers` decoder layers with real dataflow between them, M rows of x.

    Returns (stages, records, x0): records[i] = (name, stage, W fp32 host, x, q, d, N, y)
    in stage order.  Optional side linears with ragged N read inputs of their own.
    With same_sign, every weight is positive and x0 non-negative, so every
    output of the pass has |y| = sum |w_hat x| (the tightest case of the bound).
    """
    x0 = workloads.random_activations(M, hidden, seed=seed, device=gpu)
    if same_sign:
        x0 = x0.abs()
    stages, records = [], []

    def add(stage_items, name, N, K, x, wseed):
        if same_sign:
            W = (0.02 * (np.abs(np.random.default_rng(wseed).standard_normal((N, K))) + 0.25)).astype(np.float32)
        else:
            W = workloads.random_weight(N, K, std=0.02, seed=wseed)
        q, d = w4.quantize_rtn(torch.from_numpy(W).to(gpu))
        y = torch.empty((M, N), dtype=torch.bfloat16, device=gpu)
        stage_items.append((x, q, d, N, y))
        records.append((name, len(stages), W, x, q, d, N, y))
        return y

    x = x0
    for layer in range(layers):
        s = 1000 * seed + 10 * layer
        st = []
        yq = add(st, f"L{layer}.q", nq, hidden, x, s + 0)
        add(st, f"L{layer}.k", nkv, hidden, x, s + 1)
        add(st, f"L{layer}.v", nkv, hidden, x, s + 2)
        stages.append(st)
        st = []
        yo = add(st, f"L{layer}.o", hidden, nq, yq, s + 3)
        if side and layer == 0:
            add(st, "side.ragged", 77, 384, workloads.random_activations(M, 384, seed=seed + 7, device=gpu), s + 7)
        stages.append(st)
        st = []
        yg = add(st, f"L{layer}.gate", ffn, hidden, yo, s + 4)
        add(st, f"L{layer}.up", ffn, hidden, yo, s + 5)
        if side and layer == 0:
            add(st, "side.one_row", 1, 128, workloads.random_activations(M, 128, seed=seed + 8, device=gpu), s + 8)
        stages.append(st)
        st = []
        x = add(st, f"L{layer}.down", hidden, ffn, yg, s + 6)
        stages.append(st)
    return stages, records, x0


def _batched_path(M):
    """The kernel a chain of M-row linears runs, with its configuration variable."""
    return ("gemv", "W4_GEMV_CFG") if M == 1 else ("mfma", "W4_MFMA_CFG")


def _check_pass(w4, records, cfg, monkeypatch, what):
    """Bitwise against per-stage batched launches (dot2 at M = 1, unsplit MFMA
    above), and within tolerance of the oracle."""
    torch.cuda.synchronize()
    path, var = _batched_path(records[0][7].shape[0])
    monkeypatch.setenv(var, cfg)
    by_stage = {}
    for rec in records:
        by_stage.setdefault(rec[1], []).append(rec)
    for st in sorted(by_stage):
        recs = by_stage[st]
        outs = [torch.empty_like(r[7]) for r in recs]
        w4.linear_batched([(r[3], r[4], r[5], r[6], o) for r, o in zip(recs, outs)], path=path)
        for r, o in zip(recs, outs):
            assert torch.equal(r[7].view(torch.int16), o.view(torch.int16)), f"{what} {r[0]}: chain != batched"
    monkeypatch.delenv(var)
    worst = 0.0
    for name, _, W, x, _, _, _, y in records:
        q_ref, d_ref = oracle.rtn_quantize_ref(W)
        y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
        worst = max(worst, check_y(y, y_ref, absdot, f"{what} {name}"))
    return worst


@pytest.mark.parametrize("cfg", CHAIN_CFGS)
def test_chain_matches_batched_and_oracle(w4, gpu, cfg, monkeypatch):
    monkeypatch.setenv("W4_CHAIN_CFG", cfg)
    _say(f"chain cfg={cfg}: 3 layers (hidden 512, q 768, kv 256, ffn 1408) + ragged side linears")
    stages, records, x0 = _build_chain(w4, gpu, layers=3, hidden=512, nq=768, nkv=256, ffn=1408, seed=1)
    plan = w4.chain_prepare(stages)
    monkeypatch.delenv("W4_CHAIN_CFG")
    info = plan.info
    assert info["stages"] == 12 and info["linears"] == len(records)
    for rep in range(3):
        x0.copy_(workloads.random_activations(1, x0.shape[1], seed=50 + rep, device=gpu))
        plan.run()
        assert plan.error() == 0, "a chain wait timed out"
        _check_pass(w4, records, cfg, monkeypatch, f"cfg={cfg} pass {rep}")


def test_chain_same_sign_rows(w4, gpu, monkeypatch):
    """Positive weights and non-negative inputs through every stage: each output
    is the bf16 rounding of a value within the bound where the bound is tightest."""
    _say("chain with same-sign rows: 3 layers (hidden 512, q 768, kv 256, ffn 1408)")
    stages, records, x0 = _build_chain(w4, gpu, layers=3, hidden=512, nq=768, nkv=256, ffn=1408, seed=12,
                                       side=False, same_sign=True)
    plan = w4.chain_prepare(stages)
    cfg = f"{plan.plan.rows_per_item},{plan.plan.waves_per_block}"
    plan.run()
    assert plan.error() == 0, "a chain wait timed out"
    _check_pass(w4, records, cfg, monkeypatch, "same-sign")
    for name, _, W, x, *_ in records:
        assert (W > 0).all() and (x >= 0).all(), name


def test_chain_nonfinite_input_poisons_the_pass(w4, gpu, monkeypatch):
    """An infinity in the first stage's input makes every output of the pass NaN
    (each stage's input row is then non-finite); no wait times out, and every
    output equals the per-stage launches bit for bit."""
    _say("chain with an infinite input value: 2 layers")
    stages, records, x0 = _build_chain(w4, gpu, layers=2, hidden=512, nq=768, nkv=256, ffn=1408, seed=13,
                                       side=False)
    plan = w4.chain_prepare(stages)
    cfg = f"{plan.plan.rows_per_item},{plan.plan.waves_per_block}"
    x0[0, 100] = float("inf")
    plan.run()
    assert plan.error() == 0, "a chain wait timed out"
    for name, *_, y in records:
        assert torch.isnan(y).all(), f"{name}: not every output is NaN"
    _check_pass(w4, records, cfg, monkeypatch, "non-finite input")
    # and a finite input afterwards gives ordinary outputs again
    x0.copy_(workloads.random_activations(1, 512, seed=14, device=gpu))
    plan.run()
    assert plan.error() == 0
    _check_pass(w4, records, cfg, monkeypatch, "after the non-finite pass")


def test_chain_graph_replays(w4, gpu, monkeypatch):
    """Graph-captured passes replayed with eager input changes and synchronisations between them."""
    _say("chain in a HIP graph: 2 layers, 4 replays with new inputs")
    stages, records, x0 = _build_chain(w4, gpu, layers=2, hidden=1024, nq=1024, nkv=256, ffn=2816, seed=2)
    plan = w4.chain_prepare(stages)
    cfg = f"{plan.plan.rows_per_item},{plan.plan.waves_per_block}"
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        plan.run()  # warm (outside the graph)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run()
    for rep in range(4):
        x0.copy_(workloads.random_activations(1, x0.shape[1], seed=70 + rep, device=gpu))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert plan.error() == 0, "a chain wait timed out"
        _check_pass(w4, records, cfg, monkeypatch, f"graph replay {rep}")


FULL_SIZE = {"27b": (5120, 6144, 1024, 17408, 0.015), "70b": (8192, 8192, 1024, 28672, 0.01)}


@pytest.mark.parametrize("size,M", [("27b", 1), ("70b", 1), ("27b", 8), ("70b", 16)])
def test_chain_full_size_layers(w4, gpu, size, M, monkeypatch):
    """Two decoder layers at their real shapes (27B class: hidden 5120, q 6144,
    k/v 1024, ffn 17408; 70B class: hidden 8192, q 8192, k/v 1024, ffn 28672,
    the largest x a chain stages at M = 1), at decode and verification widths:
    bitwise against per-stage batched launches; oracle on sampled output rows."""
    _say(f"chain {size}-class, M={M}: 2 layers at full size")
    hidden, nq, nkv, ffn, std = FULL_SIZE[size]
    x0 = workloads.random_activations(M, hidden, seed=3, device=gpu)
    stages, records = [], []
    x = x0
    rng = np.random.default_rng(3)
    for layer in range(2):
        def mk(N, K, xin, name, st):
            W = torch.randn((N, K), device=gpu, generator=torch.Generator(gpu).manual_seed(100 * layer + len(records)))
            W.mul_(std)
            q, d = w4.quantize_rtn(W)
            rows = np.sort(rng.choice(N, size=24, replace=False))
            W_rows = W.index_select(0, torch.as_tensor(rows, device=gpu)).cpu().numpy()
            del W
            y = torch.empty((M, N), dtype=torch.bfloat16, device=gpu)
            st.append((xin, q, d, N, y))
            records.append((name, len(stages), rows, W_rows, xin, q, d, N, y))
            return y
        st = []
        yq = mk(nq, hidden, x, f"L{layer}.q", st)
        mk(nkv, hidden, x, f"L{layer}.k", st)
        mk(nkv, hidden, x, f"L{layer}.v", st)
        stages.append(st)
        st = []
        yo = mk(hidden, nq, yq, f"L{layer}.o", st)
        stages.append(st)
        st = []
        yg = mk(ffn, hidden, yo, f"L{layer}.gate", st)
        mk(ffn, hidden, yo, f"L{layer}.up", st)
        stages.append(st)
        st = []
        x = mk(hidden, ffn, yg, f"L{layer}.down", st)
        stages.append(st)
    plan = w4.chain_prepare(stages)
    cfg = f"{plan.plan.rows_per_item},{plan.plan.waves_per_block}"
    plan.run()
    assert plan.error() == 0, "a chain wait timed out"
    torch.cuda.synchronize()
    path, var = _batched_path(M)
    monkeypatch.setenv(var, cfg)
    for st_i, st in enumerate(stages):
        recs = [r for r in records if r[1] == st_i]
        outs = [torch.empty_like(r[8]) for r in recs]
        w4.linear_batched([(r[4], r[5], r[6], r[7], o) for r, o in zip(recs, outs)], path=path)
        for r, o in zip(recs, outs):
            assert torch.equal(r[8].view(torch.int16), o.view(torch.int16)), f"{r[0]}: chain != batched"
    monkeypatch.delenv(var)
    for name, _, rows, W_rows, xin, _, _, _, y in records:
        q_ref, d_ref = oracle.rtn_quantize_ref(W_rows)
        y_ref, absdot = oracle.w4_linear_ref(_bits(xin), q_ref, d_ref)
        check_y(y[:, rows], y_ref, absdot, f"{size} chain {name} (24 sampled rows)")


def test_chain_rejects_bad_chains(w4, gpu):
    _say("chain argument errors")
    W = torch.from_numpy(workloads.random_weight(32, 256, seed=4)).to(gpu)
    q, d = w4.quantize_rtn(W)
    x = workloads.random_activations(1, 256, seed=4, device=gpu)
    y = torch.empty((1, 32), dtype=torch.bfloat16, device=gpu)
    x2 = workloads.random_activations(2, 256, seed=4, device=gpu)
    y2 = torch.empty((2, 32), dtype=torch.bfloat16, device=gpu)
    x17 = workloads.random_activations(17, 256, seed=4, device=gpu)
    y17 = torch.empty((17, 32), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(w4.W4Error, match="W4_ERR_SHAPE"):
        w4.chain_prepare([[(x17, q, d, 32, y17)]])         # M is at most 16
    with pytest.raises(w4.W4Error, match="W4_ERR_SHAPE"):
        w4.chain_prepare([[(x, q, d, 32, y)], [(x2, q, d, 32, y2)]])   # one M for the whole chain
    with pytest.raises(w4.W4Error, match="W4_ERR_ARG"):
        w4.chain_prepare([[(x, q, d, 32, y), (x, q, d, 32, y)]])   # two outputs of a stage overlap
    xy = torch.empty((1, 256), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(w4.W4Error, match="W4_ERR_ARG"):
        w4.chain_prepare([[(xy, q, d, 32, xy[:, :32])]])   # y overlaps x within a stage
    # a later stage writing over an earlier stage's input (or the line it sits
    # in) is refused: the launch relies on each line being written before it
    # is read
    y_a = torch.empty((1, 256), dtype=torch.bfloat16, device=gpu)
    W2 = torch.from_numpy(workloads.random_weight(256, 256, seed=5)).to(gpu)
    q2, d2 = w4.quantize_rtn(W2)
    with pytest.raises(w4.W4Error, match="W4_ERR_ARG"):
        w4.chain_prepare([[(x, q2, d2, 256, y_a)], [(y_a, q, d, 32, y)], [(y_a, q2, d2, 256, x)]])
    # y of one stage read as x by the next: the intended use
    x_in = x.clone()
    plan = w4.chain_prepare([[(x, q2, d2, 256, y_a)], [(y_a, q, d, 32, y)]])
    plan.run()
    assert plan.error() == 0
    q_ref, d_ref = oracle.rtn_quantize_ref(W.cpu().numpy())
    q2_ref, d2_ref = oracle.rtn_quantize_ref(W2.cpu().numpy())
    for xin, (qr, dr), out, what in ((x_in, (q2_ref, d2_ref), y_a, "stage 0"), (y_a, (q_ref, d_ref), y, "stage 1")):
        y_ref, absdot = oracle.w4_linear_ref(_bits(xin), qr, dr)
        check_y(out, y_ref, absdot, what)


def test_chain_error_flag_is_sticky_until_prepare(w4, gpu, monkeypatch):
    """A pass that starts with the workspace's error flag set (as after a timed-out
    wait) stops waiting, still completes, and leaves the flag set; the next
    w4_chain_prepare clears it and passes are correct again."""
    _say("chain error flag: set from the host, pass completes, prepare clears it")
    stages, records, x0 = _build_chain(w4, gpu, layers=2, hidden=512, nq=768, nkv=256, ffn=1408, seed=6, side=False)
    plan = w4.chain_prepare(stages)
    assert plan.error() == 0
    plan.workspace[0] = 1  # the error word is the first 32 bits of the workspace
    plan.run()
    torch.cuda.synchronize()
    assert plan.error() == 1
    plan.run()
    assert plan.error() == 1
    plan = w4.chain_prepare(stages)
    assert plan.error() == 0
    plan.run()
    assert plan.error() == 0
    cfg = f"{plan.plan.rows_per_item},{plan.plan.waves_per_block}"
    _check_pass(w4, records, cfg, monkeypatch, "after prepare")


@pytest.mark.parametrize("M", [1, 8])
def test_chain_16bit_scales(w4, gpu, M, monkeypatch):
    """The chained pass with bf16 scales: bitwise equal to per-stage batched
    launches with 16-bit scales in the same configuration, and within tolerance
    of the oracle's 16-bit-scale quantization, over two passes with new inputs."""
    _say(f"chain with 16-bit scales, M={M}: 2 layers + ragged side linears")
    x0 = workloads.random_activations(M, 512, seed=9, device=gpu)
    stages, records = [], []

    def add(st, name, N, K, x, wseed):
        W = workloads.random_weight(N, K, std=0.02, seed=wseed)
        q, d = w4.quantize_rtn(torch.from_numpy(W).to(gpu), scale_dtype=torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=gpu)
        st.append((x, q, d, N, y))
        records.append((name, len(stages), W, x, q, d, N, y))
        return y

    x = x0
    for layer in range(2):
        s = 500 + 10 * layer
        st = []
        yq = add(st, f"L{layer}.q", 768, 512, x, s)
        add(st, f"L{layer}.k", 256, 512, x, s + 1)
        stages.append(st)
        st = []
        yo = add(st, f"L{layer}.o", 512, 768, yq, s + 2)
        if layer == 0:
            add(st, "side.ragged", 77, 384, workloads.random_activations(M, 384, seed=11, device=gpu), s + 7)
        stages.append(st)
        st = []
        yg = add(st, f"L{layer}.gate", 1408, 512, yo, s + 3)
        add(st, f"L{layer}.up", 1408, 512, yo, s + 4)
        stages.append(st)
        st = []
        x = add(st, f"L{layer}.down", 512, 1408, yg, s + 5)
        stages.append(st)
    plan = w4.chain_prepare(stages)
    assert plan.info["scale_bytes"] == 2
    cfg = f"{plan.plan.rows_per_item},{plan.plan.waves_per_block}"
    path, var = _batched_path(M)
    for rep in range(2):
        x0.copy_(workloads.random_activations(M, 512, seed=90 + rep, device=gpu))
        plan.run()
        assert plan.error() == 0
        torch.cuda.synchronize()
        monkeypatch.setenv(var, cfg)
        for st_i in range(len(stages)):
            recs = [r for r in records if r[1] == st_i]
            outs = [torch.empty_like(r[7]) for r in recs]
            w4.linear_batched([(r[3], r[4], r[5], r[6], o) for r, o in zip(recs, outs)], path=path)
            for r, o in zip(recs, outs):
                assert torch.equal(r[7].view(torch.int16), o.view(torch.int16)), f"pass {rep} {r[0]}: chain != batched"
        monkeypatch.delenv(var)
        for name, _, W, xin, _, _, _, y in records:
            q_ref, d_ref = oracle.rtn_quantize_ref(W, "bf16")
            y_ref, absdot = oracle.w4_linear_ref(_bits(xin), q_ref, d_ref)
            check_y(y, y_ref, absdot, f"s16 chain pass {rep} {name}")


# ---------------------------------------------------------------------------
# verification widths (M = 2..16): MFMA items
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,M", [(c, m) for c in CHAIN_MFMA_CFGS for m in (8, 16)] +
                         [("2,4", 2), ("2,4", 5), ("4,4", 13), ("1,4", 3)])
def test_chain_verify_matches_batched_and_oracle(w4, gpu, cfg, M, monkeypatch):
    monkeypatch.setenv("W4_CHAIN_CFG", cfg)
    _say(f"chain cfg={cfg} M={M}: 3 layers (hidden 512, q 768, kv 256, ffn 1408) + ragged side linears")
    stages, records, x0 = _build_chain(w4, gpu, layers=3, hidden=512, nq=768, nkv=256, ffn=1408, seed=21, M=M)
    plan = w4.chain_prepare(stages)
    monkeypatch.delenv("W4_CHAIN_CFG")
    info = plan.info
    assert info["stages"] == 12 and info["linears"] == len(records) and info["x_rows"] == M
    assert f"{plan.plan.rows_per_item},{plan.plan.waves_per_block}" == cfg
    for rep in range(3):
        x0.copy_(workloads.random_activations(M, x0.shape[1], seed=150 + rep, device=gpu))
        plan.run()
        assert plan.error() == 0, "a chain wait timed out"
        _check_pass(w4, records, cfg, monkeypatch, f"cfg={cfg} M={M} pass {rep}")


def test_chain_verify_same_sign_rows(w4, gpu, monkeypatch):
    _say("chain M=8 with same-sign rows: 3 layers (hidden 512, q 768, kv 256, ffn 1408)")
    stages, records, x0 = _build_chain(w4, gpu, layers=3, hidden=512, nq=768, nkv=256, ffn=1408, seed=22,
                                       side=False, same_sign=True, M=8)
    plan = w4.chain_prepare(stages)
    cfg = f"{plan.plan.rows_per_item},{plan.plan.waves_per_block}"
    plan.run()
    assert plan.error() == 0, "a chain wait timed out"
    _check_pass(w4, records, cfg, monkeypatch, "M=8 same-sign")


def test_chain_verify_nonfinite_row(w4, gpu, monkeypatch):
    """An infinity in row 3 of the first stage's input: row 3 of every output of
    the pass is NaN (each stage's row 3 reads only the previous stage's row 3),
    every other row is finite and correct, and no wait times out."""
    _say("chain M=8 with an infinite input value in row 3: 2 layers")
    stages, records, x0 = _build_chain(w4, gpu, layers=2, hidden=512, nq=768, nkv=256, ffn=1408, seed=23,
                                       side=False, M=8)
    plan = w4.chain_prepare(stages)
    cfg = f"{plan.plan.rows_per_item},{plan.plan.waves_per_block}"
    x0[3, 100] = float("inf")
    plan.run()
    assert plan.error() == 0, "a chain wait timed out"
    for name, *_, y in records:
        assert torch.isnan(y[3]).all(), f"{name}: row 3 is not all NaN"
        assert torch.isfinite(y[torch.arange(8, device=y.device) != 3]).all(), f"{name}: another row is not finite"
    _check_pass(w4, records, cfg, monkeypatch, "M=8 non-finite row")


def test_chain_verify_graph_replays(w4, gpu, monkeypatch):
    """M = 16 passes captured in a graph and replayed with new inputs."""
    _say("chain M=16 in a HIP graph: 2 layers, 4 replays with new inputs")
    stages, records, x0 = _build_chain(w4, gpu, layers=2, hidden=1024, nq=1024, nkv=256, ffn=2816, seed=24, M=16)
    plan = w4.chain_prepare(stages)
    cfg = f"{plan.plan.rows_per_item},{plan.plan.waves_per_block}"
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        plan.run()  # warm (outside the graph)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run()
    for rep in range(4):
        x0.copy_(workloads.random_activations(16, x0.shape[1], seed=170 + rep, device=gpu))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert plan.error() == 0, "a chain wait timed out"
        _check_pass(w4, records, cfg, monkeypatch, f"M=16 graph replay {rep}")


def test_chain_verify_error_flag_is_sticky_until_prepare(w4, gpu, monkeypatch):
    _say("chain M=8 error flag: set from the host, pass completes, prepare clears it")
    stages, records, x0 = _build_chain(w4, gpu, layers=2, hidden=512, nq=768, nkv=256, ffn=1408, seed=25,
                                       side=False, M=8)
    plan = w4.chain_prepare(stages)
    plan.workspace[0] = 1
    plan.run()
    assert plan.error() == 1
    plan = w4.chain_prepare(stages)
    plan.run()
    assert plan.error() == 0
    cfg = f"{plan.plan.rows_per_item},{plan.plan.waves_per_block}"
    _check_pass(w4, records, cfg, monkeypatch, "M=8 after prepare")


def test_chain_verify_noalloc(w4, gpu, monkeypatch):
    """M = 8 set up in the library's static scratch (w4_chain_prepare_noalloc):
    the same pass as with a caller-owned workspace, bit for bit."""
    _say("chain M=8 prepared in the static scratch (noalloc): 2 layers")
    stages, records, x0 = _build_chain(w4, gpu, layers=2, hidden=512, nq=768, nkv=256, ffn=1408, seed=27,
                                       side=False, M=8)
    plan = w4.chain_prepare(stages, noalloc=True)
    assert plan.info["x_rows"] == 8
    plan.run()
    assert plan.error() == 0
    cfg = f"{plan.plan.rows_per_item},{plan.plan.waves_per_block}"
    _check_pass(w4, records, cfg, monkeypatch, "M=8 noalloc")


@pytest.mark.parametrize("M", [1, 8])
def test_chain_trace_timestamps(w4, gpu, M, monkeypatch):
    """w4_chain_trace: every item gets a start and an end stamp in order, and at
    M = 1 an input-staged stamp between them (0 for items that reused the
    previous item's input; always 0 at M > 1); the outputs are those of an
    untraced pass bit for bit, and clearing it stops the writes."""
    # (K of 2048 and more: every wavefront of an item has a scale quad of its own)
    _say(f"chain timestamps M={M}: 2 layers (hidden 2048)")
    stages, records, x0 = _build_chain(w4, gpu, layers=2, hidden=2048, nq=2048, nkv=512, ffn=2816, seed=28,
                                       side=False, M=M)
    plan = w4.chain_prepare(stages)
    plan.run()
    torch.cuda.synchronize()
    ref = [r[7].clone() for r in records]
    items = plan.plan.items
    stamps = torch.zeros(3 * items + 3, dtype=torch.int64, device=gpu)
    plan.trace(stamps)
    plan.run()
    assert plan.error() == 0
    for r, y in zip(records, ref):
        assert torch.equal(r[7].view(torch.int16), y.view(torch.int16)), f"{r[0]}: traced pass differs"
    t = stamps.cpu().numpy()
    assert t[-3:].tolist() == [0, 0, 0], "wrote past the items"
    t = t[:-3].reshape(items, 3)
    start, ready, end = t[:, 0], t[:, 1], t[:, 2]
    assert (start > 0).all() and (end >= start).all()
    waited = ready > 0
    assert ((ready[waited] >= start[waited]) & (ready[waited] <= end[waited])).all()
    assert waited.any() if M == 1 else not waited.any()
    assert plan.plan.trace == 1
    plan.trace(None)
    assert plan.plan.trace == 0
    stamps.zero_()
    plan.run()
    assert plan.error() == 0
    assert int(stamps.abs().sum()) == 0
