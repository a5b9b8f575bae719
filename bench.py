"""Benchmark of the W4A16 decode linear on one MI355X.

Headline (the JSON line's `value`): achieved algorithmic HBM bandwidth of one
decode step's linear layers on the 70B-class stack (hidden 8192, FFN 28672,
80 layers: q/k/v, o, gate/up and down of every layer, 36.4 GB of 4-bit codes
and fp32 scales per pass) at M = 1, run as ONE chained launch that keeps the
layer's dependencies (w4_chain_run: q|k|v read the previous layer's down
output, o reads q, gate|up read o, down reads gate).  Every pass reads every
weight once, so it streams from HBM.  One step = one pass; exactly --steps
passes are timed after --warmup passes (and at least 150 ms of warmup), replayed
from a HIP graph, with events on the replay stream bracketed by
synchronisations.

Reported beside it in the same line: the same stack at M = 8 (verifying 7
drafted tokens + 1) in the fastest launch mode that keeps the dependencies;
the roofline of the chained kernel; the CPU oracle timed on this host's cores
(a sequential phase after the GPU work); and, as extra keys, the 4B- and
27B-class stacks in every launch mode, the 2560x9216 / 9216x2560 pair one
launch per linear and batched, quantization throughput, 16-bit scales, and the
channel-scaling (AWQ) and GPTQ quantizers.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--stacks 4b,27b,70b|none] [--no-cpu]
"""

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "w4_linear achieved HBM GB/s (% of peak) at M=1 and M=8; equiv decode tok/s"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E nameplate
PEAK_BF16_FLOPS = 2.5e15  # MI355X dense bf16 MFMA
HEADLINE = "stack_70b"    # the largest configuration: the 70B-class layer stack
PAIR = "ffn_pair_outliers"
KERNEL_SOURCES = ["bit_group_quantized_w4_amd/csrc/linear.hip", "bit_group_quantized_w4_amd/csrc/w4_device.h",
                  "bit_group_quantized_w4_amd/csrc/w4_launch.h"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "linear_chain_stack_70b_m1_counters.json")
HEADLINE_KERNEL = "linear_chain_kernel"  # the persistent chained pass (one dispatch per pass)
BENCH_SUPPORT = os.path.join(ROOT, "bench_support")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the headline kernel's source code: comments and whitespace are
    dropped, so that editing a comment does not retire the stored counters."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------
# GPU timing helpers
# ----------------------------------------------------------------------------

def capture(torch, fn, reps=1):
    """Capture `reps` back-to-back calls of fn() (library launches) into one HIP graph."""
    fn()  # eager run first: nothing lazy happens inside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    return g


def graph_steps(steps):
    """Steps per graph replay: the largest of 8, 4, 2, 1 dividing `steps`, so
    that exactly `steps` steps are timed while replay overhead is amortized."""
    for r in (8, 4, 2, 1):
        if steps % r == 0:
            return r
    return 1


# Under sustained load the GPU's clocks settle only after tens of milliseconds:
# replays of the headline launch run ~117 us, then ~180 us, then recover to a
# steady ~121 us after about 40 ms.  Warmup therefore lasts at least this long.
MIN_WARMUP_S = 0.15


def time_graph(torch, g, replays, warmup):
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < MIN_WARMUP_S:
        g.replay()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()  # keep the host from running far ahead of the clock check
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3  # seconds


# ----------------------------------------------------------------------------
# headline: single-matrix pair, weight copies rotated through HBM
# ----------------------------------------------------------------------------

def bench_pair(torch, w4, workloads, steps, warmup, copies, scale_dtype=None, ms=None, quantize=True):
    """The 2560x9216 / 9216x2560 pair: each of `copies` weight copies of both
    matrices multiplied once per step, one launch per linear and batched."""
    dev = torch.device("cuda:0")
    wl = workloads.WORKLOADS[PAIR]
    scale_dtype = scale_dtype or torch.float32
    sb = 2 if scale_dtype == torch.bfloat16 else 4
    tag = "" if sb == 4 else " (16-bit scales)"
    mats = []
    for m in wl.matrices:
        W = torch.from_numpy(workloads.weight(PAIR, 0, m.name, "cpu")).to(dev)
        q0, d0 = w4.quantize_rtn(W, scale_dtype=scale_dtype)
        qs = [q0] + [q0.clone() for _ in range(copies - 1)]
        ds = [d0] + [d0.clone() for _ in range(copies - 1)]
        mats.append((m, W, qs, ds))
    torch.cuda.synchronize()
    out = {}
    for M in (ms or wl.ms):
        xs = [workloads.activations(PAIR, 0, m.name, M, dev) for (m, _, _, _) in mats]
        ys = [torch.empty((M, m.N), dtype=torch.bfloat16, device=dev) for (m, _, _, _) in mats]
        # batched mode: every linear of a step writes its own output
        ysb = [[torch.empty((M, m.N), dtype=torch.bfloat16, device=dev) for (m, _, _, _) in mats]
               for _ in range(copies)]
        ws = w4.SplitWorkspace(dev) if M > 1 else None

        def step():
            for c in range(copies):
                for i, (m, _, qs, ds) in enumerate(mats):
                    w4.linear(xs[i], qs[c], ds[c], m.N, out=ys[i], workspace=ws)

        def step_batched():
            items = [(xs[i], qs[c], ds[c], m.N, ysb[c][i])
                     for c in range(copies) for i, (m, _, qs, ds) in enumerate(mats)]
            for b in range(0, len(items), w4.MAX_BATCH):
                w4.linear_batched(items[b:b + w4.MAX_BATCH], workspace=ws)

        step_bytes = copies * sum(workloads.algorithmic_bytes(M, m.N, m.K, sb) for (m, _, _, _) in mats)
        res = {}
        for mode, fn in (("per_call", step), ("batched", step_batched)):
            gs = graph_steps(steps)
            g = capture(torch, fn, gs)
            t = time_graph(torch, g, steps // gs, max(1, warmup // gs))
            launches = steps * (copies * len(mats) if mode == "per_call"
                                else -(-copies * len(mats) // w4.MAX_BATCH))
            gbs = steps * step_bytes / t / 1e9
            res[mode] = {
                "GBps": round(gbs, 1),
                "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
                "us_per_launch": round(t / launches * 1e6, 3),
                "us_per_linear": round(t / (steps * copies * len(mats)) * 1e6, 3),
                "ms_per_step": round(t / steps * 1e3, 4),
                "launches_per_step": launches // steps,
            }
            log(f"[bench] {PAIR}{tag} M={M} {mode}: {gbs:.0f} GB/s, "
                f"{t / (steps * copies * len(mats)) * 1e6:.2f} us per linear")
            del g
        res["bytes_per_call"] = {m.name: workloads.algorithmic_bytes(M, m.N, m.K, sb) for (m, _, _, _) in mats}
        out[M] = res
    # quantization throughput (rows a1-a4), same matrices, rotated over 4 fp32 copies
    qout = {}
    nq = min(4, copies)
    for (m, W, qs, ds) in (mats if quantize else []):
        Ws = [W] + [W.clone() for _ in range(nq - 1)]

        def qstep():
            for c in range(nq):
                w4.quantize_rtn(Ws[c], out=(qs[c], ds[c]))

        g = capture(torch, qstep)
        t = time_graph(torch, g, max(3, steps // 4), 2)
        n = max(3, steps // 4) * nq
        qb = workloads.quantize_bytes(m.N, m.K, sb)
        qout[m.name] = {"GBps": round(n * qb / t / 1e9, 1), "us_per_call": round(t / n * 1e6, 2),
                        "bytes_per_call": qb}
        log(f"[bench] quantize {m.name} {m.N}x{m.K}: {n * qb / t / 1e9:.0f} GB/s")
        del g, Ws
    if quantize:
        # one full-size 70B-class gate matrix (28672 x 8192, 0.94 GB of fp32
        # weights): the size the quantizer meets when a large model is converted
        m = next(mm for mm in workloads.WORKLOADS["stack_70b"].matrices if mm.name == "gate")
        Wg = workloads.weight("stack_70b", 0, "gate", dev)
        qg, dg = w4.quantize_rtn(Wg, scale_dtype=scale_dtype)
        g = capture(torch, lambda: w4.quantize_rtn(Wg, out=(qg, dg)))
        n = max(3, steps // 16)
        t = time_graph(torch, g, n, 2)
        qb = workloads.quantize_bytes(m.N, m.K, sb)
        qout["stack_70b_gate"] = {"GBps": round(n * qb / t / 1e9, 1), "us_per_call": round(t / n * 1e6, 2),
                                  "bytes_per_call": qb}
        log(f"[bench] quantize 70B gate {m.N}x{m.K}: {n * qb / t / 1e9:.0f} GB/s")
        del g, Wg, qg, dg
    del mats
    torch.cuda.empty_cache()
    return out, qout


# ----------------------------------------------------------------------------
# layer stacks: one graph = one decode (or verify) pass over every linear
# ----------------------------------------------------------------------------

def _shared_input_groups(wl):
    """Matrices of one layer grouped by the input they read (q|k|v, o, gate|up, down)."""
    order, by_tag = [], {}
    for i, m in enumerate(wl.matrices):
        tag = wl.input_groups.get(m.name, m.name)
        if tag not in by_tag:
            by_tag[tag] = []
            order.append(tag)
        by_tag[tag].append(i)
    return [by_tag[t] for t in order]


def bench_stack(torch, w4, workloads, name, steps, warmup, only_ms=None, only_modes=None, scale_dtype=None,
                chain_steps=None, chain_warmup=None):
    dev = torch.device("cuda:0")
    wl = workloads.WORKLOADS[name]
    scale_dtype = scale_dtype or torch.float32
    sb = 2 if scale_dtype == torch.bfloat16 else 4
    t0 = time.time()
    layers = []
    for layer in range(wl.layers):
        mats = []
        for m in wl.matrices:
            W = workloads.weight(name, layer, m.name, dev)
            q, d = w4.quantize_rtn(W, scale_dtype=scale_dtype)
            del W
            mats.append((m, q, d))
        layers.append(mats)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"[bench] stack {name}: {wl.layers} layers quantized in {time.time() - t0:.1f}s")
    res = {}
    groups = {"per_call": [[i] for i in range(len(wl.matrices))],
              "fused_shared_input": _shared_input_groups(wl),
              "layer_batched": [list(range(len(wl.matrices)))]}
    if only_modes:
        groups = {k: v for k, v in groups.items() if k in only_modes}
    for M in wl.ms:
        if only_ms and M not in only_ms:
            continue
        xs = {m.K: workloads.activations(name, 0, m.name, M, dev) for m in wl.matrices}
        ys = [torch.empty((M, m.N), dtype=torch.bfloat16, device=dev) for m in wl.matrices]
        # verification widths: the MFMA kernel may split a launch's K across blocks
        ws = w4.SplitWorkspace(dev) if M > 1 else None
        res[M] = {}
        for mode, grp in groups.items():
            def step():
                for mats in layers:
                    for gi in grp:
                        if len(gi) == 1:
                            m, q, d = mats[gi[0]]
                            w4.linear(xs[m.K], q, d, m.N, out=ys[gi[0]], workspace=ws)
                        else:
                            w4.linear_batched([(xs[mats[i][0].K], mats[i][1], mats[i][2], mats[i][0].N, ys[i])
                                               for i in gi], workspace=ws)

            g = capture(torch, step)
            t = time_graph(torch, g, steps, warmup)
            per = t / steps
            nbytes = workloads.stack_bytes(name, M, sb)
            gbs = nbytes / per / 1e9
            flops = 2.0 * M * workloads.stack_weights(name)
            res[M][mode] = {"ms_per_pass": round(per * 1e3, 4), "GBps": round(gbs, 1),
                            "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
                            "passes_per_s": round(1 / per, 2), "tokens_per_s_ceiling": round(M / per, 1),
                            "launches_per_pass": len(layers) * len(grp),
                            "useful_tflops": round(flops / per / 1e12, 2),
                            "pct_of_bf16_mfma_peak": round(100 * flops / per / PEAK_BF16_FLOPS, 3)}
            log(f"[bench] stack {name}{'' if sb == 4 else ' (16-bit scales)'} M={M} {mode}: {per * 1e3:.3f} ms/pass, {gbs:.0f} GB/s, "
                f"{1 / per:.1f} passes/s")
            del g
        if not only_modes or "chained" in only_modes:
            res[M]["chained"] = bench_chain(torch, w4, workloads, wl, layers, xs, chain_steps or steps,
                                            chain_warmup or warmup, name, sb, M)
        res[M]["bytes_per_pass"] = workloads.stack_bytes(name, M, sb)
    del layers
    torch.cuda.empty_cache()
    return res


# launch modes that keep a decode layer's dependencies (o after q|k|v, down after gate|up)
DEPENDENT_MODES = ("per_call", "fused_shared_input", "chained")


def decode_summary(stacks):
    """Per stack at M = 1: the fastest launch mode that keeps the layer's
    dependencies, as equivalent decode tokens/s of the linear layers (1 / pass
    time) and % of the 8 TB/s roofline; the independent-launch upper bound
    beside it."""
    out = {}
    for name, res in stacks.items():
        m1 = res.get(1) or res.get("1") or {}
        dep = {k: v for k, v in m1.items() if k in DEPENDENT_MODES}
        if not dep:
            continue
        mode, best = min(dep.items(), key=lambda kv: kv[1]["ms_per_pass"])
        entry = {"mode": mode, "tokens_per_s": round(1e3 / best["ms_per_pass"], 1), "ms_per_pass": best["ms_per_pass"],
                 "GBps": best["GBps"], "pct_of_peak": best["pct_of_peak"]}
        if "layer_batched" in m1:
            entry["upper_bound_independent_launches"] = {"tokens_per_s": round(1e3 / m1["layer_batched"]["ms_per_pass"], 1),
                                                         "pct_of_peak": m1["layer_batched"]["pct_of_peak"]}
        out[name] = entry
    return out


# Mean tokens accepted per verification pass of seven drafted tokens (M = 8), as the
# 27B quantization-and-drafter ladder page reports them for its drafter (stage 2): 2.2-2.5
# on prose, 5.3-5.6 on code.  Used only for the illustrative rates of verify_summary.
ACCEPTANCE_M8 = {"prose": (2.2, 2.5), "code": (5.3, 5.6)}


def verify_summary(stacks):
    """Per stack at each M > 1: the fastest launch mode that keeps the layer's
    dependencies, as passes/s and the ceiling M / T_pass (every drafted token
    accepted); at M = 8 also the illustrative tokens/s tau / T_pass at the
    acceptance lengths above (linear layers only, drafter cost not included)."""
    out = {}
    for name, res in stacks.items():
        for M, modes in res.items():
            if not isinstance(modes, dict) or int(M) <= 1:
                continue
            dep = {k: v for k, v in modes.items() if k in DEPENDENT_MODES and isinstance(v, dict)}
            if not dep:
                continue
            mode, best = min(dep.items(), key=lambda kv: kv[1]["ms_per_pass"])
            passes = 1e3 / best["ms_per_pass"]
            entry = {"mode": mode, "ms_per_pass": best["ms_per_pass"], "pct_of_peak": best["pct_of_peak"],
                     "passes_per_s": round(passes, 1), "ceiling_tokens_per_s": round(int(M) * passes, 1)}
            if int(M) == 8:
                entry["tokens_per_s_at_acceptance"] = {k: [round(t * passes, 1) for t in v]
                                                       for k, v in ACCEPTANCE_M8.items()}
            out.setdefault(name, {})[int(M)] = entry
    return out


def chain_stages(torch, wl, layers, xs, M, dev=None):
    """The stages of a chained pass over a stack: the shared-input groups of
    every layer, each stage reading the output of the previous one (q|k|v <-
    previous down, o <- q, gate|up <- o, down <- gate); the first stage reads
    xs[K].  layers: per layer, (matrix, q, d) in the stack's matrix order.
    Outputs are allocated on `dev` (default cuda:0).
    Returns (stages for w4.chain_prepare, the kind of each stage)."""
    dev = dev if dev is not None else torch.device("cuda:0")
    groups = _shared_input_groups(wl)
    stages, kinds, prev = [], [], []  # prev: (N, y) of the previous stage's linears
    for mats in layers:
        # outputs of every layer in buffers of their own: a chain writes each line once
        ys = {m.name: torch.empty((M, m.N), dtype=torch.bfloat16, device=dev) for m in wl.matrices}
        for gi in groups:
            K = mats[gi[0]][0].K
            x = next((y for n, y in prev if n == K), xs[K])
            stages.append([(x, mats[i][1], mats[i][2], mats[i][0].N, ys[mats[i][0].name]) for i in gi])
            kinds.append("|".join(mats[i][0].name for i in gi))
            prev = [(mats[i][0].N, ys[mats[i][0].name]) for i in gi]
    return stages, kinds


def bench_chain(torch, w4, workloads, wl, layers, xs, steps, warmup, name, scale_bytes=4, M=1):
    """One pass of the whole stack at M rows of x (a decode step at M = 1, the
    verification of M - 1 drafted tokens above) as one chained launch
    (w4_chain_run) over the stages of chain_stages, as in a real pass."""
    stages, _ = chain_stages(torch, wl, layers, xs, M)
    plan = w4.chain_prepare(stages)
    g = capture(torch, plan.run)
    t = time_graph(torch, g, steps, warmup)
    err = plan.error()
    if err:
        raise RuntimeError(f"{name} chained pass: a wait timed out (error flag {err}); the timing is invalid")
    per = t / steps
    nbytes = workloads.stack_bytes(name, M, scale_bytes)
    gbs = nbytes / per / 1e9
    flops = 2.0 * M * workloads.stack_weights(name)
    out = {"ms_per_pass": round(per * 1e3, 4), "GBps": round(gbs, 1), "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
           "passes_per_s": round(1 / per, 2), "tokens_per_s_ceiling": round(M / per, 1), "launches_per_pass": 1,
           "stages_per_pass": len(stages), "useful_tflops": round(flops / per / 1e12, 2),
           "pct_of_bf16_mfma_peak": round(100 * flops / per / PEAK_BF16_FLOPS, 3),
           "plan": plan.info, "wait_timeouts": err, "timed_passes": steps}
    log(f"[bench] stack {name}{'' if scale_bytes == 4 else ' (16-bit scales)'} M={M} chained: {per * 1e3:.3f} ms/pass, {gbs:.0f} GB/s, {1 / per:.1f} passes/s "
        f"(plan {plan.info}, timeouts {err})")
    del g, plan
    return out


def chain_stage_times(torch, w4, workloads, name, M, passes=3):
    """Where a chained pass spends its time, stage by stage (w4_chain_trace).

    The stack's chain at M (as bench_chain builds it) runs `passes` eager
    passes; the last one is traced.  Per kind of stage (q|k|v, o, gate|up,
    down), averaged over the layers: its items, the stage's span (from the end
    of the previous stage's last item to the end of its own last item), when
    its first item had its input relative to the previous stage's end, the
    items' mean and longest duration from input to end, and the share of the
    grid's blocks that held one of its items.  Times in microseconds.  Only
    the M = 1 kernel stamps when an item had its input; at M > 1
    ("timed_from": "start") both figures count from the item's start, so an
    item's duration includes its wait for the input.
    """
    import numpy as np

    dev = torch.device("cuda:0")
    wl = workloads.WORKLOADS[name]
    layers = []
    for layer in range(wl.layers):
        mats = []
        for m in wl.matrices:
            W = workloads.weight(name, layer, m.name, dev)
            q, d = w4.quantize_rtn(W)
            del W
            mats.append((m, q, d))
        layers.append(mats)
    xs = {m.K: workloads.activations(name, 0, m.name, M, dev) for m in wl.matrices}
    stages, kinds = chain_stages(torch, wl, layers, xs, M)
    plan = w4.chain_prepare(stages)
    items = plan.plan.items
    stamps = torch.zeros(3 * items, dtype=torch.int64, device=dev)
    for p in range(passes):
        if p == passes - 1:
            plan.trace(stamps)
        plan.run()
    if plan.error():
        raise RuntimeError(f"{name} chained pass: a wait timed out")
    plan.trace(None)
    t = stamps.cpu().numpy().reshape(items, 3).astype(np.int64)
    # item ranges of the stages, from the chain's table (item0 and stage of each linear)
    n = plan.plan.linears
    tab = plan.workspace[32:32 + 64 * n].cpu().numpy().view(np.int32).reshape(n, 16)
    # the table's entries (w4_launch.h ChainLinear: a 48-byte LinearDesc whose
    # int32 words 8-11 are M, K, N, flags, then item0 and stage) must be the
    # chain's linears, stage by stage, their items in order
    if not (tab[0, 12] == 0 and np.all(np.diff(tab[:, 12]) >= 0) and np.all(np.diff(tab[:, 13]) >= 0)
            and tab[-1, 13] == len(stages) - 1):
        raise RuntimeError("chain table layout: item and stage columns are not where expected")
    for si, st in enumerate(stages):
        got = sorted((int(k), int(nn)) for k, nn, s_ in zip(tab[:, 9], tab[:, 10], tab[:, 13]) if s_ == si)
        if got != sorted((int(x.shape[1]), int(N)) for x, _, _, N, _ in st):
            raise RuntimeError(f"chain table layout: stage {si} does not hold the stage's linears")
    first = {}
    for item0, st in zip(tab[:, 12], tab[:, 13]):
        first[int(st)] = min(first.get(int(st), items), int(item0))
    bounds = [first[s] for s in range(len(stages))] + [items]
    T0 = t[:, 0].min()
    prev_end = T0
    acc = {}
    for s, kind in enumerate(kinds):
        a, b = bounds[s], bounds[s + 1]
        st = t[a:b]
        end = st[:, 2].max()
        ready = st[:, 1][st[:, 1] > 0]
        first_ready = ready.min() if len(ready) else st[:, 0].min()
        dur = st[:, 2] - np.maximum(st[:, 0], st[:, 1])
        r = acc.setdefault(kind, {"items": b - a, "span": [], "ready": [], "mean": [], "max": []})
        r["span"].append((end - prev_end) * 0.01)
        r["ready"].append((first_ready - prev_end) * 0.01)
        r["mean"].append(dur.mean() * 0.01)
        r["max"].append(dur.max() * 0.01)
        prev_end = end
    total = (t[:, 2].max() - T0) * 0.01
    out = {"workload": name, "M": M, "items": items, "blocks": plan.plan.blocks, "rows_per_item": plan.plan.rows_per_item * 16,
           "waves_per_block": plan.plan.waves_per_block, "traced_pass_us": round(float(total), 1),
           "timed_from": "input" if (t[:, 1] > 0).any() else "start", "stages": {}}
    for kind, r in acc.items():
        out["stages"][kind] = {"items": r["items"], "span_us": round(float(np.mean(r["span"])), 2),
                               "first_input_after_prev_end_us": round(float(np.mean(r["ready"])), 2),
                               "item_mean_us": round(float(np.mean(r["mean"])), 2),
                               "item_max_us": round(float(np.mean(r["max"])), 2),
                               "grid_share": round(min(1.0, r["items"] / plan.plan.blocks), 3)}
    del plan, layers
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------
# channel scaling before RTN (AWQ): the exponent search and the fused decode linear
# ----------------------------------------------------------------------------

def bench_awq(torch, w4, workloads, steps, warmup, T=256):
    """On the 70B-class gate matrix (28672x8192, layer 0) with calibration rows drawn
    from the same recipe: the search time and the output error relative to RTN, for
    the recipe as is (its salient input channels also carry x20 weights) and for the
    same matrix with those weight columns left ordinary; then the decode linear at
    M = 1 with x/s formed in the kernel's staging against the plain linear."""
    from bit_group_quantized_w4_amd import awq

    dev = torch.device("cuda:0")
    name, mat = "stack_70b", "gate"
    W = workloads.weight(name, 0, mat, dev)
    N, K = W.shape
    x_cal = workloads.activations(name, 0, mat, T, dev)
    chans = workloads.outlier_channels(name, 0, workloads.WORKLOADS[name].input_groups.get(mat, mat), K)
    mult = workloads.WORKLOADS[name].weight[4]
    x_eval = workloads.activations(name, 0, mat, 1024, dev)  # held-out rows: an independent draw
    out = {"matrix": f"{N}x{K}", "calibration_rows": T, "held_out_rows": x_eval.shape[0]}
    for tag, Wv in (("recipe", W), ("ordinary_weights_on_salient_channels", None)):
        if Wv is None:
            Wv = W.clone()
            Wv[:, torch.as_tensor(chans, device=dev)] /= mult
        awq.search(Wv, x_cal)  # warm
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        res = awq.search(Wv, x_cal)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        e = res["errors"]
        # the chosen scaling against plain RTN on rows the search never saw
        y_ref = torch.matmul(x_eval.float(), Wv.t())
        q0, d0 = w4.quantize_rtn(Wv)
        e_awq = float(w4.sq_error(w4.linear(w4.scale_activations(x_eval, res["inv_s"]), res["q"], res["d"], N),
                                  y_ref).item())
        e_rtn = float(w4.sq_error(w4.linear(x_eval, q0, d0, N), y_ref).item())
        del y_ref, q0, d0
        out[tag] = {"k": res["k"], "alpha": round(res["alpha"], 4), "error_vs_rtn": round(e[res["k"]] / e[0], 4),
                    "held_out_error_vs_rtn": round(e_awq / e_rtn, 4), "search_ms": round(dt * 1e3, 1)}
        log(f"[bench] awq {tag}: alpha={res['alpha']:.3f}, output error {e[res['k']] / e[0]:.3f} x RTN "
            f"(held-out rows {e_awq / e_rtn:.3f}), search {dt * 1e3:.0f} ms")
    # decode: fused x/s staging against the plain linear, same matrix, rotated copies
    res = awq.search(W, x_cal)
    copies = 8
    qs = [res["q"].clone() for _ in range(copies)]
    ds = [res["d"].clone() for _ in range(copies)]
    x = workloads.activations(name, 0, mat, 1, dev)
    y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
    nbytes = copies * workloads.algorithmic_bytes(1, N, K) + copies * 4 * K  # + inv_s
    for mode in ("linear_awq", "linear"):
        def step():
            for c in range(copies):
                if mode == "linear_awq":
                    w4.linear_awq(x, qs[c], ds[c], N, res["inv_s"], out=y)
                else:
                    w4.linear(x, qs[c], ds[c], N, out=y)
        g = capture(torch, step)
        t = time_graph(torch, g, max(4, steps // 8), warmup)
        per = t / (max(4, steps // 8) * copies)
        out[mode + "_m1"] = {"us_per_call": round(per * 1e6, 2), "GBps": round(nbytes / copies / per / 1e9, 1)}
        del g
    log(f"[bench] awq decode M=1: fused {out['linear_awq_m1']['GBps']:.0f} GB/s, plain {out['linear_m1']['GBps']:.0f} GB/s")
    del W, qs, ds
    torch.cuda.empty_cache()
    return out


# Path comparison: both linear kernels, one launch per linear, on a short-K and a
# long-K matrix; eight weight copies rotated so every launch streams from HBM.
PC_SHAPES = ((2560, 9216), (28672, 8192))
PC_MS = (1, 2, 3, 4, 8, 16)
PC_PATHS = ("gemv", "mfma")
PC_STEPS = 64
PC_COPIES = 8


def path_compare(torch, w4, workloads):
    """Both linear kernels on the same matrices at M = 1..4, 8 and 16: the evidence
    behind the automatic path choice (dot2 at M = 1, MFMA from M = 2).  Logs one line
    per (shape, M) and returns the rows; the timed dispatches are the last
    PC_STEPS * PC_COPIES of each (shape, M, path) in a kernel trace."""
    dev = torch.device("cuda:0")
    rows = []
    copies = PC_COPIES
    for (N, K) in PC_SHAPES:
        W = torch.from_numpy(workloads.random_weight(N, K, seed=N + K)).to(dev)
        q0, d0 = w4.quantize_rtn(W)
        del W
        qs = [q0] + [q0.clone() for _ in range(copies - 1)]
        ds = [d0] + [d0.clone() for _ in range(copies - 1)]
        for M in PC_MS:
            x = workloads.random_activations(M, K, seed=M, device=dev)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            res = {}
            for path in PC_PATHS:
                def step():
                    for c in range(copies):
                        w4.linear(x, qs[c], ds[c], N, path=path, out=y)
                g = capture(torch, step)
                t = time_graph(torch, g, PC_STEPS, 4) / (PC_STEPS * copies)
                res[path] = round(workloads.algorithmic_bytes(M, N, K) / t / 1e9, 1)
                del g
            rows.append({"N": N, "K": K, "M": M, **res})
            log(f"[bench] path compare {N}x{K} M={M}: dot2 {res['gemv']:.0f} GB/s, MFMA {res['mfma']:.0f} GB/s")
        del qs, ds
        torch.cuda.empty_cache()
    return rows


def bench_gptq(torch, w4, workloads, T=16384, T_eval=1024):
    """GPTQ of the 70B-class gate matrix (28672x8192, layer 0) calibrated on T rows
    (T = 2K, so the Hessian is well determined): time per phase, and the output error
    against RTN's (both through the library's linear) on the calibration rows and on
    T_eval held-out rows, for two input recipes:
      * "recipe": the 70B recipe's activations, whose channels are independent
        (diagonal covariance), so column feedback can only fit the sample
        Hessian's noise;
      * "correlated": the same rows mixed by one fixed matrix A = I + 2 G / sqrt(K)
        (G standard normal, seeded), so the channels are strongly correlated."""
    from bit_group_quantized_w4_amd import gptq

    dev = torch.device("cuda:0")
    name, mat = "stack_70b", "gate"
    W = workloads.weight(name, 0, mat, dev)
    N, K = W.shape
    q_rtn, d_rtn = w4.quantize_rtn(W)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20)
    A = torch.randn((K, K), generator=gen, device=dev).mul_(2.0 / K ** 0.5)
    A.diagonal().add_(1.0)
    out = {"matrix": f"{N}x{K}", "calibration_rows": T, "held_out_rows": T_eval}
    for case in ("recipe", "correlated"):
        x_cal = workloads.activations(name, 0, mat, T, dev)
        x_eval = workloads.activations(name, 0, mat, T_eval, dev)
        if case == "correlated":
            x_cal = (x_cal.float() @ A).to(torch.bfloat16)
            x_eval = (x_eval.float() @ A).to(torch.bfloat16)
        if case == "recipe":
            gptq.quantize(W, x_cal)  # warm: libraries load their kernels
        torch.cuda.synchronize()
        tm = {}
        t0 = time.perf_counter()
        q, d = gptq.quantize(W, x_cal, timings=tm)
        torch.cuda.synchronize()
        total = time.perf_counter() - t0
        ratios = {}
        for rows, x in (("calibration", x_cal[:T_eval]), ("held_out", x_eval)):
            y_ref = torch.matmul(x.float(), W.t())
            e = {tag: float(w4.sq_error(w4.linear(x, qq, dd, N), y_ref).item())
                 for tag, (qq, dd) in (("gptq", (q, d)), ("rtn", (q_rtn, d_rtn)))}
            ratios[rows] = round(e["gptq"] / e["rtn"], 4)
            del y_ref
        out[case] = {"ms_total": round(total * 1e3, 1), "ms_phases": {k: round(v, 2) for k, v in tm.items()},
                     "output_error_vs_rtn": ratios}
        log(f"[bench] gptq {N}x{K} {case} (T={T}): {total * 1e3:.0f} ms "
            f"({', '.join(f'{k} {v:.1f}' for k, v in tm.items())} ms), output error x RTN: "
            f"calibration rows {ratios['calibration']:.3f}, held-out rows {ratios['held_out']:.3f}")
        del q, d, x_cal, x_eval
    del W, A
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------
# CPU oracle baseline (bounded sample, rank 0, after the GPU phase)
# ----------------------------------------------------------------------------

def host_cores():
    """Cores this process may run on; on hosts that give a GPU a share of the CPU
    (OMP_NUM_THREADS set), that share."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(omp)) if omp.isdigit() and int(omp) > 0 else n


def cpu_baseline(workloads, budget_s=20.0):
    """The CPU oracle as it stands (oracle.w4_linear_ref: fp64 dequantization, then a
    BLAS product), timed after the GPU phase on this host's cores:

    * the headline workload's M = 1 pass, estimated from each distinct matrix shape
      of a 70B-class layer timed once and summed over its multiplicity and the 80
      layers (all cores: BLAS threads pinned to the core count; NumPy's elementwise
      steps run on one thread);
    * the 2560 x 9216 matrix at M = 1 on one core, and the quantizer on it
      (oracle.rtn_quantize_ref; the weights are drawn before the clock starts).

    Codes and scales are drawn at random for the timing (the oracle's cost does not
    depend on their values)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    cores = host_cores()
    wl = workloads.WORKLOADS[HEADLINE]
    rng = np.random.default_rng(0)
    shapes = {}
    for m in wl.matrices:
        shapes.setdefault((m.N, m.K), []).append(m.name)
    per_shape = {}
    t_layer = 0.0
    with threadpool_limits(limits=cores):
        for (N, K), names in shapes.items():
            q = rng.integers(-7, 8, (N, K), dtype=np.int8)
            d = rng.uniform(1e-3, 1e-2, (N, K // 128)).astype(np.float32)
            x = (rng.standard_normal((1, K), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
            oracle.w4_linear_ref(x[:, :128], q[:16, :128], d[:16, :1])  # warm the BLAS threads
            t0 = time.perf_counter()
            oracle.w4_linear_ref(x, q, d)
            t = time.perf_counter() - t0
            per_shape[f"{N}x{K}"] = {"seconds": round(t, 3), "matrices_per_layer": len(names)}
            t_layer += t * len(names)
            del q, d
    t_pass = t_layer * wl.layers
    nbytes = workloads.stack_bytes(HEADLINE, 1)
    # one core, the 2560 x 9216 matrix: the linear and the quantizer
    N, K = 2560, 9216
    W = workloads.weight("ffn_2560x9216", 0, "ffn", "cpu")
    x1 = workloads.activations("ffn_2560x9216", 0, "ffn", 1, "cpu").view(-1).view(__import__("torch").int16).numpy()
    x1 = x1.view(np.uint16).reshape(1, K)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        q1, d1 = oracle.rtn_quantize_ref(W)
        tq = time.perf_counter() - t0
        n1, t0 = 0, time.perf_counter()
        while n1 < 3 or time.perf_counter() - t0 < budget_s / 4:
            oracle.w4_linear_ref(x1, q1, d1)
            n1 += 1
        t1 = (time.perf_counter() - t0) / n1
    b1 = workloads.algorithmic_bytes(1, N, K)
    return {"value": round(nbytes / t_pass / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"70B-class stack at M = 1: each distinct matrix shape of a layer timed once with "
                      f"oracle.w4_linear_ref ({', '.join(per_shape)}), summed over its matrices and the "
                      f"{wl.layers} layers; BLAS on {cores} threads, NumPy's elementwise steps on one",
            "seconds_per_pass_estimated": round(t_pass, 2), "equiv_decode_tokens_per_s": round(1 / t_pass, 5),
            "per_shape": per_shape,
            "one_core_2560x9216_m1": {"GBps": round(b1 / t1 / 1e9, 4), "ms_per_call": round(t1 * 1e3, 1),
                                      "calls": n1, "cores": 1},
            "one_core_quantize_2560x9216": {"GBps": round(workloads.quantize_bytes(N, K) / tq / 1e9, 4),
                                            "seconds": round(tq, 2), "cores": 1}}


# ----------------------------------------------------------------------------

def bench_lib():
    """bench_support/libw4_bench.so (measurement-only kernels), built if missing."""
    import ctypes
    import importlib.util

    path = os.path.join(BENCH_SUPPORT, "libw4_bench.so")
    if not os.path.exists(path):
        spec = importlib.util.spec_from_file_location("w4_bench_build", os.path.join(BENCH_SUPPORT, "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build(verbose=False)
    return ctypes.CDLL(path)


def measure_read_peak(torch, w4, gib=4, reps=5):
    """Bandwidth of a plain streaming read (grid-stride, non-temporal 16-byte loads) over
    `gib` GiB on this GPU: the practical ceiling for a kernel that only reads."""
    import ctypes

    lib = bench_lib()
    nb = gib << 30
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    grid = 2048
    sink = torch.zeros(grid, dtype=torch.int32, device="cuda:0")

    def run():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert lib.w4bench_read(ctypes.c_void_p(buf.data_ptr()), ctypes.c_int64(nb),
                                ctypes.c_void_p(sink.data_ptr()), grid, s) == 0

    g = capture(torch, run, reps)
    t = time_graph(torch, g, 2, 1) / (2 * reps)
    del g, buf
    torch.cuda.empty_cache()
    gbs = nb / t / 1e9
    log(f"[bench] streaming read peak: {gbs:.0f} GB/s")
    return {"GBps": round(gbs, 1), "pct_of_nameplate": round(100 * gbs / PEAK_HBM_GBS, 2),
            "kernel": "grid-stride read, non-temporal 16-byte loads, 2048 blocks of 256 threads",
            "bytes": nb}


def roofline(chained, bytes_per_pass, read_peak=None):
    """Dominant kernel: the chained pass over the 70B-class stack at M = 1 (one
    dispatch of the persistent kernel per pass, after a small fill launch).
    achieved = algorithmic bytes per pass / the pass time measured with events
    on the replay stream over the timed passes (the fill launch, ~5 us, is
    inside that time)."""
    achieved = round(bytes_per_pass / (chained["ms_per_pass"] * 1e-3) / 1e9, 1)
    traffic = None
    if os.path.exists(COUNTERS_FILE):
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
        if c.get("kernel_source_hash") == kernel_source_hash():
            traffic = c.get("hbm_bytes_per_launch")
    p = chained.get("plan", {})
    return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
            "kernel": f"{HEADLINE_KERNEL}<{p.get('rows_per_item', 32) // 16}, {p.get('waves_per_block')}, false> "
                      f"(persistent dot2 pass, {p.get('blocks')} blocks), one dispatch per pass",
            "algorithmic_bytes_per_launch": bytes_per_pass,
            "avg_launch_us": round(chained["ms_per_pass"] * 1e3, 1),
            "frac_of_measured_read_peak": round(achieved / read_peak["GBps"], 4) if read_peak else None,
            "traffic_source": "rocprofv3 FETCH_SIZE + WRITE_SIZE of this kernel, copy-kernel calibrated"
                              if traffic else None}


# ----------------------------------------------------------------------------
# rocprofv3 output summaries (used to write the text files under profiles/)
# ----------------------------------------------------------------------------

def summarize_trace(path, last=0):
    """Per (kernel, grid, block) duration statistics from a rocprofv3 kernel_trace.csv.
    With `last`, also the mean duration of the last `last` dispatches of the
    headline kernel (the timed passes of a run that times only the 70B-class
    chained pass, e.g. --stacks 70b --stack-ms 1 --stack-modes chained)."""
    import csv
    import statistics

    rows = list(csv.DictReader(open(path)))
    if last:
        head = sorted((r for r in rows if HEADLINE_KERNEL in r["Kernel_Name"]), key=lambda r: int(r["Start_Timestamp"]))
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in head]
        tail = d[-last:]
        print(f"headline {HEADLINE_KERNEL}: {len(d)} dispatches; "
              f"last {len(tail)} (the timed passes): mean {statistics.mean(tail):.2f} us, "
              f"median {statistics.median(tail):.2f} us, min {min(tail):.2f} us, max {max(tail):.2f} us\n")
    groups = {}
    for r in rows:
        name = r["Kernel_Name"].replace("w4::(anonymous namespace)::", "")
        key = (name[:70], int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])), int(r["Grid_Size_Y"]),
               int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    print("| kernel | blocks | grid y | block | calls | avg us | median us | min us | max us |")
    print("|---|---|---|---|---|---|---|---|---|")
    for key, v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| {key[0]} | {key[1]} | {key[2]} | {key[3]} | {len(v)} | {statistics.mean(v) / 1e3:.2f} | "
              f"{statistics.median(v) / 1e3:.2f} | {min(v) / 1e3:.2f} | {max(v) / 1e3:.2f} |")


def summarize_path_compare(path):
    """Per-case kernel durations of a `--path-compare` run from its kernel_trace.csv.
    Dispatches are split into runs of one (kernel, grid); the runs of linear kernels
    long enough to hold a timed case are matched, in order, with the cases
    path_compare runs, and the last PC_STEPS * PC_COPIES dispatches of each are used."""
    import csv
    import statistics

    import workloads

    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    runs = []
    for r in rows:
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if runs and runs[-1][0] == key:
            runs[-1][1].append(dur)
        else:
            runs.append((key, [dur]))
    timed = PC_STEPS * PC_COPIES
    runs = [(k, v) for k, v in runs if "linear_" in k[0] and len(v) >= timed]
    cases = [(N, K, M, p) for (N, K) in PC_SHAPES for M in PC_MS for p in PC_PATHS]
    if len(runs) != len(cases):
        raise SystemExit(f"expected {len(cases)} timed runs of linear kernels, found {len(runs)}")
    print("| N x K | M | path | kernel | blocks | timed dispatches | mean us | median us | GB/s (mean) |")
    print("|---|---|---|---|---|---|---|---|---|")
    best = {}
    for (N, K, M, p), ((name, blocks), v) in zip(cases, runs):
        t = v[-timed:]
        mean = statistics.mean(t) / 1e3
        gbs = workloads.algorithmic_bytes(M, N, K) / (mean * 1e-6) / 1e9
        best.setdefault((N, K, M), {})[p] = gbs
        name = name.replace("w4::(anonymous namespace)::", "")
        print(f"| {N}x{K} | {M} | {'dot2' if p == 'gemv' else 'MFMA'} | {name[:60]} | {blocks} | {len(t)} | "
              f"{mean:.2f} | {statistics.median(t) / 1e3:.2f} | {gbs:.0f} |")
    print()
    print("| N x K | M | dot2 GB/s | MFMA GB/s | faster |")
    print("|---|---|---|---|---|")
    for (N, K, M), r in best.items():
        print(f"| {N}x{K} | {M} | {r['gemv']:.0f} | {r['mfma']:.0f} | "
              f"{'dot2' if r['gemv'] > r['mfma'] else 'MFMA'} ({max(r.values()) / min(r.values()):.2f}x) |")


def summarize_counters(path):
    """Mean of each counter per (kernel, grid) from a rocprofv3 counter_collection.csv."""
    import csv
    import statistics

    groups = {}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"].replace("w4::(anonymous namespace)::", "")[:70]
        grid = int(r.get("Grid_Size", r.get("Grid_Size_X", 0)))
        groups.setdefault((name, grid, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    print("| kernel | grid (threads) | counter | dispatches | mean per dispatch |")
    print("|---|---|---|---|---|")
    for (name, grid, cn), v in sorted(groups.items()):
        print(f"| {name} | {grid} | {cn} | {len(v)} | {statistics.mean(v):.1f} |")


def write_counters(fetch_csv, write_csv, copy_mb, out_path):
    """Traffic of the headline kernel from two rocprofv3 --pmc runs of
    `bench.py --calibrate-copy-mb copy_mb` that time only the 70B-class chained
    pass (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the
    same counter reads for the plain copy kernel of known size."""
    import csv
    import statistics

    import workloads

    def per_dispatch(path, counter):
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    copy_bytes = copy_mb << 20
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        d = per_dispatch(path, counter)
        copy = [v for k, v in d.items() if "copy_kernel" in k]
        factor = statistics.mean(copy[0]) * 1024 / copy_bytes  # counter bytes per real byte
        vals = [v for k, v in d.items() if HEADLINE_KERNEL in k]
        if not vals:
            raise SystemExit(f"no {HEADLINE_KERNEL} dispatch in {path}")
        kib = statistics.median(vals[0])
        res[counter] = {"kib_per_dispatch": kib, "dispatches": len(vals[0]),
                        "copy_calibration_factor": round(factor, 4), "bytes_per_dispatch": round(kib * 1024 / factor)}
    traffic = res["FETCH_SIZE"]["bytes_per_dispatch"] + res["WRITE_SIZE"]["bytes_per_dispatch"]
    out = {"kernel": HEADLINE_KERNEL, "launch": "one chained pass over the 70B-class stack at M = 1 (80 layers)",
           "kernel_source_hash": kernel_source_hash(), "counters": res,
           "hbm_bytes_per_launch": traffic,
           "algorithmic_bytes_per_launch": workloads.stack_bytes(HEADLINE, 1)}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--copies", type=int, default=32)
    ap.add_argument("--stacks", default="4b,27b,70b",
                    help="stacks measured besides the headline 70B-class stack (always measured)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-pair", action="store_true",
                    help="skip the 2560x9216 / 9216x2560 pair, its quantization and the read peak (profiling runs)")
    ap.add_argument("--no-awq", action="store_true", help="skip the channel-scaling (AWQ) search and decode timing")
    ap.add_argument("--no-s16", action="store_true", help="skip the 16-bit-scale measurements")
    ap.add_argument("--no-gptq", action="store_true", help="skip the GPTQ quantizer measurement")
    ap.add_argument("--path-compare", action="store_true",
                    help="only time both linear kernels at M = 1..4, 8, 16 (profiling runs)")
    ap.add_argument("--stack-ms", default="", help="comma list: only these M for the stacks (profiling runs)")
    ap.add_argument("--stack-modes", default="",
                    help="comma list of per_call, fused_shared_input, layer_batched, chained (profiling runs)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="also run the plain copy kernel on this many MiB (counter calibration)")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="print a duration summary of a rocprofv3 kernel trace and exit")
    ap.add_argument("--trace-last", type=int, default=0,
                    help="with --trace-summary: mean of the last N headline dispatches (the timed steps)")
    ap.add_argument("--path-compare-summary", metavar="KERNEL_TRACE_CSV",
                    help="per-case kernel durations of a --path-compare run")
    ap.add_argument("--chain-stage-times", metavar="STACK:M",
                    help="per-stage times of one traced chained pass (e.g. stack_27b:1) as a JSON line, and exit")
    ap.add_argument("--counter-summary", metavar="COUNTER_COLLECTION_CSV",
                    help="print a summary of a rocprofv3 counter collection and exit")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files into the traffic file and exit")
    args = ap.parse_args()

    if args.write_counters:
        write_counters(args.write_counters[0], args.write_counters[1], args.calibrate_copy_mb or 256,
                       COUNTERS_FILE)
        return
    if args.path_compare_summary:
        summarize_path_compare(args.path_compare_summary)
        return
    if args.trace_summary:
        summarize_trace(args.trace_summary, args.trace_last)
        return
    if args.counter_summary:
        summarize_counters(args.counter_summary)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(no sharding or collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_group_quantized_w4_amd as w4
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.init()

    if args.path_compare:
        print(json.dumps({"path_compare": path_compare(torch, w4, workloads)}), flush=True)
        return
    if args.chain_stage_times:
        name, M = args.chain_stage_times.split(":")
        print(json.dumps({"chain_stage_times": chain_stage_times(torch, w4, workloads, name, int(M))}), flush=True)
        return

    only_ms = [int(m) for m in args.stack_ms.split(",") if m] or None
    only_modes = [m for m in args.stack_modes.split(",") if m] or None

    # The headline: the 70B-class stack, its chained M = 1 pass timed over exactly
    # --steps passes (the other launch modes and M over a fifth of that).
    stacks = {HEADLINE: bench_stack(torch, w4, workloads, HEADLINE, max(5, args.steps // 5), max(2, args.warmup),
                                    only_ms, only_modes, chain_steps=args.steps, chain_warmup=args.warmup)}
    for s in [s for s in args.stacks.split(",") if s and s != "none" and "stack_" + s != HEADLINE]:
        stacks["stack_" + s] = bench_stack(torch, w4, workloads, "stack_" + s, max(5, args.steps // 5),
                                           max(2, args.warmup), only_ms, only_modes)

    pair = quant = None
    if not args.no_pair:
        pair, quant = bench_pair(torch, w4, workloads, args.steps, args.warmup, args.copies)

    # 16-bit scales: the pair at M = 1 and the stacks at M = 1 in the two launch modes that keep
    # a layer's dependencies (one launch per stage, chained)
    s16 = None
    if not args.no_s16:
        s16 = {} if args.no_pair else {"pair": bench_pair(torch, w4, workloads, args.steps, args.warmup, args.copies,
                                                          scale_dtype=torch.bfloat16, ms=[1], quantize=False)[0]}
        for name in stacks:
            s16[name] = bench_stack(torch, w4, workloads, name, max(5, args.steps // 5), max(2, args.warmup), [1],
                                    ["fused_shared_input", "chained"], scale_dtype=torch.bfloat16)

    awq_res = None if args.no_awq else bench_awq(torch, w4, workloads, args.steps, args.warmup)
    gptq_res = None if args.no_gptq else bench_gptq(torch, w4, workloads)
    read_peak = None if args.no_pair else measure_read_peak(torch, w4)

    if args.calibrate_copy_mb:
        import ctypes

        lib = bench_lib()
        nb = args.calibrate_copy_mb << 20
        a = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
        b = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for _ in range(3):
            assert lib.w4bench_copy(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                    ctypes.c_int64(nb), 2048, s) == 0
        torch.cuda.synchronize()
        log(f"[bench] copy kernel: 3 x {args.calibrate_copy_mb} MiB")

    torch.cuda.synchronize()
    # CPU phase: after every GPU measurement, never overlapped with one
    cpu = None if args.no_cpu else cpu_baseline(workloads)

    wl = workloads.WORKLOADS[HEADLINE]
    head_res = stacks[HEADLINE].get(1, {})
    head = head_res.get("chained")
    if head is None:
        print(json.dumps({"stacks": stacks}), flush=True)  # a profiling run without the chained pass
        return
    nbytes = workloads.stack_bytes(HEADLINE, 1)
    dec = decode_summary(stacks)
    m8 = stacks[HEADLINE].get(8, {})
    m8_dep = {k: v for k, v in m8.items() if k in DEPENDENT_MODES}
    m8_best = min(m8_dep.items(), key=lambda kv: kv[1]["ms_per_pass"]) if m8_dep else None
    line = {
        "metric": METRIC,
        "value": head["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_pass"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "layers": wl.layers,
                   "matrices_per_layer": {m.name: f"{m.N}x{m.K}" for m in wl.matrices},
                   "M": 1, "linears_per_pass": wl.layers * len(wl.matrices), "stages_per_pass": head["stages_per_pass"],
                   "launch": "w4_chain_run: the whole dependent pass as one persistent launch (after a fill launch)",
                   "group": 128, "weights": "int4 codes + fp32 scales", "x": "bf16",
                   "bytes_per_pass": nbytes,
                   "timing": "hip graph replay of one pass per step, events on the replay stream",
                   "min_warmup_ms": int(MIN_WARMUP_S * 1000)},
        "pct_of_peak": head["pct_of_peak"],
        "equiv_decode_tokens_per_s": round(1e3 / head["ms_per_pass"], 1),
        "m8": ({"mode": m8_best[0], **m8_best[1],
                "bytes_per_pass": m8.get("bytes_per_pass")} if m8_best else None),
        "decode_summary": dec,
        "verify_summary": verify_summary(stacks),
        "roofline": roofline(head, nbytes, read_peak),
        "hbm_read_peak_measured": read_peak,
        "stacks": stacks,
        "pair": pair,
        "per_call_m1": pair[1]["per_call"] if pair else None,
        "quantize": quant,
        "scales_16bit": s16,
        "awq": awq_res,
        "gptq": gptq_res,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
