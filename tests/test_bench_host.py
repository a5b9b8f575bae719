"""Host-side logic of bench.py (no GPU): the one-GPU contract, graph step
grouping, the source hash that keys stored counters, and the copy-kernel
calibration of the HBM byte counters."""

import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_graph_steps_divides_the_timed_steps(bench):
    for steps in range(1, 130):
        r = bench.graph_steps(steps)
        assert r in (1, 2, 4, 8) and steps % r == 0
        assert all(steps % c for c in (1, 2, 4, 8) if c > r)


def test_source_hash_ignores_comments_only(bench, tmp_path, monkeypatch):
    code = "__global__ void k(int* p) {\n  p[0] = 1;  // store\n}\n"
    f = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["k.hip"])
    f.write_text(code)
    h0 = bench.kernel_source_hash()
    f.write_text("/* a new\n   block comment */\n" + code.replace("// store", "// a different comment"))
    assert bench.kernel_source_hash() == h0
    f.write_text(code.replace("p[0] = 1", "p[0] = 2"))
    assert bench.kernel_source_hash() != h0


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, grid, value in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter, "Counter_Value": value})


def test_counters_are_scaled_by_the_copy_kernel(bench, tmp_path, monkeypatch):
    mb = 256
    copy_bytes = mb << 20
    fetch_factor, read, written = 0.5, 803_000_000, 753_664
    head = f"void w4::{bench.HEADLINE_KERNEL}<2, 4, false>(w4::ChainLinear const*, unsigned int*, int)"
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [
        ("copy_kernel(x)", 524288, fetch_factor * copy_bytes / 1024),
        (head, 131072, fetch_factor * read / 1024),
        (head, 131072, fetch_factor * read / 1024),
        (head, 131072, fetch_factor * (read + 4096) / 1024),  # an outlier: the median is taken
        ("other_kernel", 1024, 123.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [
        ("copy_kernel(x)", 524288, copy_bytes / 1024),
        (head, 131072, written / 1024)])
    out = tmp_path / "counters.json"
    bench.write_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), mb, str(out))
    res = json.load(open(out))
    assert res["counters"]["FETCH_SIZE"]["bytes_per_dispatch"] == read
    assert res["counters"]["WRITE_SIZE"]["bytes_per_dispatch"] == written
    assert res["hbm_bytes_per_launch"] == read + written
    assert res["kernel"] == bench.HEADLINE_KERNEL
    assert res["counters"]["FETCH_SIZE"]["dispatches"] == 3


def test_path_compare_summary_matches_runs_to_cases(bench, tmp_path, capsys):
    timed = bench.PC_STEPS * bench.PC_COPIES
    cases = [(N, K, M, p) for (N, K) in bench.PC_SHAPES for M in bench.PC_MS for p in bench.PC_PATHS]
    fields = ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"]
    t = 0
    rows = []

    def dispatch(name, grid, dur):
        nonlocal t
        rows.append({"Kernel_Name": name, "Grid_Size_X": grid, "Workgroup_Size_X": 256,
                     "Start_Timestamp": t, "End_Timestamp": t + dur})
        t += dur + 10

    for i, (N, K, M, p) in enumerate(cases):
        if M == bench.PC_MS[0] and p == bench.PC_PATHS[0]:
            for _ in range(3):
                dispatch("quantize_kernel", 4096, 500)  # a short run of a non-linear kernel
        name = f"linear_{p}_kernel<{i}>"
        for _ in range(40):
            dispatch(name, 256 * 100, 99_000)  # eager run and warmup: excluded
        for _ in range(timed):
            dispatch(name, 256 * 100, 1000 + i)  # the timed dispatches: 1 us + i ns
    with open(tmp_path / "trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        w.writerows(rows[::-1])  # order must come from the timestamps
    bench.summarize_path_compare(str(tmp_path / "trace.csv"))
    out = capsys.readouterr().out
    lines = [ln for ln in out.splitlines() if ln.startswith("| ") and "kernel<" in ln]
    assert len(lines) == len(cases)
    for i, ln in enumerate(lines):
        cells = [c.strip() for c in ln.strip("|").split("|")]
        N, K, M, p = cases[i]
        assert cells[0] == f"{N}x{K}" and cells[1] == str(M)
        assert cells[4] == "100" and cells[5] == str(timed)
        assert float(cells[6]) == pytest.approx((1000 + i) / 1e3, abs=0.006)
    # the comparison table names the faster path: MFMA runs always end 1 ns later here
    assert out.count("| dot2 (") == len(bench.PC_SHAPES) * len(bench.PC_MS)


def test_path_compare_summary_rejects_a_short_trace(bench, tmp_path):
    with open(tmp_path / "trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp",
                                           "End_Timestamp"])
        w.writeheader()
        w.writerow({"Kernel_Name": "linear_gemv_kernel<0>", "Grid_Size_X": 256, "Workgroup_Size_X": 256,
                    "Start_Timestamp": 0, "End_Timestamp": 1000})
    with pytest.raises(SystemExit):
        bench.summarize_path_compare(str(tmp_path / "trace.csv"))


def test_decode_summary_takes_the_fastest_dependent_mode(bench):
    """Equivalent decode tokens/s come from a launch mode that keeps the layer's
    dependencies; the independent-launch upper bound is reported beside it, never
    instead of it."""
    m = lambda ms, pct: {"ms_per_pass": ms, "GBps": 1.0, "pct_of_peak": pct}
    stacks = {"stack_x": {1: {"per_call": m(4.0, 10), "fused_shared_input": m(3.0, 20), "chained": m(2.5, 30),
                              "layer_batched": m(2.0, 40)}, 8: {"fused_shared_input": m(1.0, 90)}},
              "stack_y": {"1": {"per_call": m(5.0, 10), "fused_shared_input": m(4.0, 20)}}}
    s = bench.decode_summary(stacks)
    assert s["stack_x"]["mode"] == "chained" and s["stack_x"]["tokens_per_s"] == 400.0
    assert s["stack_x"]["upper_bound_independent_launches"]["tokens_per_s"] == 500.0
    assert s["stack_y"]["mode"] == "fused_shared_input" and "upper_bound_independent_launches" not in s["stack_y"]


def test_verify_summary_rates(bench):
    """At M > 1 the fastest dependency-keeping mode gives passes/s and the ceiling
    M / T; at M = 8 also tau / T for the acceptance lengths the drafter page reports."""
    m = lambda ms: {"ms_per_pass": ms, "GBps": 1.0, "pct_of_peak": 50.0}
    stacks = {"stack_x": {1: {"chained": m(1.0)},
                          8: {"per_call": m(4.0), "fused_shared_input": m(2.0), "layer_batched": m(1.0)},
                          16: {"fused_shared_input": m(2.5)}}}
    s = bench.verify_summary(stacks)["stack_x"]
    assert 1 not in s
    assert s[8]["mode"] == "fused_shared_input" and s[8]["passes_per_s"] == 500.0
    assert s[8]["ceiling_tokens_per_s"] == 4000.0
    assert s[8]["tokens_per_s_at_acceptance"] == {"prose": [1100.0, 1250.0], "code": [2650.0, 2800.0]}
    assert s[16]["ceiling_tokens_per_s"] == 6400.0 and "tokens_per_s_at_acceptance" not in s[16]


@pytest.mark.parametrize("name", ["stack_4b", "stack_27b", "stack_70b"])
def test_chain_stages_wire_each_stage_to_the_previous_output(bench, name):
    """The chained pass bench.py times: per layer the stages q|k|v, o, gate|up,
    down; the first reads the external input, every later one the output of
    the previous stage with matching width (q|k|v <- the previous layer's
    down, o <- q, gate|up <- o, down <- gate)."""
    import torch

    import workloads

    wl = workloads.WORKLOADS[name]
    layers = [[(m, None, None) for m in wl.matrices] for _ in range(3)]
    dev = torch.device("meta")
    xs = {m.K: torch.empty((1, m.K), dtype=torch.bfloat16, device=dev) for m in wl.matrices}
    stages, kinds = bench.chain_stages(torch, wl, layers, xs, 1, dev=dev)
    assert kinds == ["q|k|v", "o", "gate|up", "down"] * 3
    mats = {m.name: m for m in wl.matrices}
    out = {}  # (stage, matrix name) -> y
    for s, (st, kind) in enumerate(zip(stages, kinds)):
        names = kind.split("|")
        assert [N for _, _, _, N, _ in st] == [mats[n].N for n in names]
        for n, (x, _, _, N, y) in zip(names, st):
            assert x.shape == (1, mats[n].K) and y.shape == (1, N)
            out[(s, n)] = y
        x = st[0][0]
        assert all(item[0] is x for item in st), "a stage's linears share one input"
        if s == 0:
            assert x is xs[mats["q"].K]
        else:
            feeder = {"q|k|v": "down", "o": "q", "gate|up": "o", "down": "gate"}[kind]
            assert x is out[(s - 1, feeder)], f"stage {s} ({kind}) must read {feeder} of stage {s - 1}"
    ys = [y for st in stages for *_, y in st]
    assert len({id(y) for y in ys}) == len(ys), "every linear writes a buffer of its own"
