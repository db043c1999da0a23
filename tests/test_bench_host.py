"""Host-side checks of the benchmark's profile summaries (no GPU): the counter
summary's calibration against the known-size copy and the record it keeps per
configuration, and the kernel-trace summary's split of a trace into decode steps."""
import argparse
import csv
import json
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

COLS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _pmc(path, counter, dispatches):
    """dispatches: (kernel name, [values summed per dispatch])."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for d, (name, vals) in enumerate(dispatches):
            for v in vals:   # a derived counter may come as several rows
                w.writerow({"Correlation_Id": d, "Dispatch_Id": d, "Kernel_Name": name,
                            "Counter_Name": counter, "Counter_Value": v})


def test_counter_summary_calibrates_and_records(tmp_path, monkeypatch, capsys):
    traffic = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    score = "void prism::(anonymous namespace)::score_anchor_kernel<4, 4>(prism::Geometry, int)"
    merge = "void prism::(anonymous namespace)::merge_kernel<4>(prism::Geometry, int)"
    other = "void at::native::fill_kernel(int)"
    # the copy: 1 MiB read and written; FETCH_SIZE reports half the bytes read
    _pmc(tmp_path / "cf.csv", "FETCH_SIZE", [("copy", [256.0, 256.0]), (other, [0.1])])
    _pmc(tmp_path / "cw.csv", "WRITE_SIZE", [("copy", [1024.0]), (other, [0.1])])
    _pmc(tmp_path / "f.csv", "FETCH_SIZE",
         [(score, [100.0, 28.0]), (score, [120.0, 8.0]), (merge, [2.0]), (other, [5.0])])
    _pmc(tmp_path / "w.csv", "WRITE_SIZE", [(score, [4.0]), (score, [4.0]), (merge, [1.0]),
                                            (other, [5.0])])
    bj = tmp_path / "bench.json"
    bj.write_text("[bench] log line\n" + json.dumps(
        {"kernels": {"anchor_score": {"algorithmic_bytes_per_launch": 262144},
                     "merge": {"avg_us": 1.0}}}) + "\n")
    args = argparse.Namespace(counter_summary=[str(tmp_path / n) for n in
                                               ("f.csv", "w.csv", "cf.csv", "cw.csv")],
                              copy_probe_mib=1, bench_json=str(bj), workload="tiny-4k-gqa4",
                              pool_rho=0, int2=False, pattern="", dense=False)
    bench.counter_summary(args)
    out = capsys.readouterr().out
    assert "scaled by 2.0000" in out and "by 1.0000" in out
    # 128 KiB fetched x 2 + 4 KiB written = 266240 bytes per dispatch
    row = [l for l in out.splitlines() if "score_anchor_kernel<4, 4>" in l][0]
    assert "| anchor_score | 2 | 128.0 | 4.0 | 2.662e+05 | 2.621e+05 | 1.016 |" in row
    assert not [l for l in out.splitlines() if "at::native" in l]
    rec = json.loads(traffic.read_text())
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()
    e = rec["kernels"]["anchor_score"]["tiny-4k-gqa4"]
    assert e["hbm_bytes_per_launch"] == 266240 and e["dispatches_averaged"] == 2
    assert "merge" not in rec["kernels"]   # no algorithmic bytes: not recorded
    assert bench.traffic_for("anchor_score", "tiny-4k-gqa4") == 266240
    assert bench.traffic_for("anchor_score", "llama3-8b-32k") is None
    # a second workload, and an option that changes the traffic, are added
    # beside the first; a run of that configuration only finds its own record
    args.workload = "llama3-8b-32k"
    bench.counter_summary(args)
    args.int2, args.pool_rho = True, 4
    bench.counter_summary(args)
    rec = json.loads(traffic.read_text())
    assert set(rec["kernels"]["anchor_score"]) == {"tiny-4k-gqa4", "llama3-8b-32k",
                                                   "llama3-8b-32k/rho4/int2"}
    assert bench.traffic_for("anchor_score", bench.config_key(args)) == 266240
    args.int2 = False
    assert bench.traffic_for("anchor_score", bench.config_key(args)) is None


def test_counter_summary_needs_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    _pmc(tmp_path / "cf.csv", "FETCH_SIZE", [("copy", [10.0])])   # far below 1 GiB
    _pmc(tmp_path / "x.csv", "FETCH_SIZE", [])
    args = argparse.Namespace(counter_summary=[str(tmp_path / n) for n in
                                               ("x.csv", "x.csv", "cf.csv", "cf.csv")],
                              copy_probe_mib=1024, bench_json="", workload="tiny-4k-gqa4",
                              pool_rho=0, int2=False, pattern="", dense=False)
    with pytest.raises(SystemExit):
        bench.counter_summary(args)


def test_trace_summary_splits_steps(tmp_path, capsys, monkeypatch):
    import synth
    wl = synth.BY_NAME["tiny-4k-gqa4"]
    per_step = bench.launches_per_step(wl, 256, 0, bench.layer_roles(wl))
    n = sum(per_step.values())
    W, K = 1, 3
    total = (W + max(1, W)) * n + 2 * K * n + n   # warm-ups, two regions, byte pass
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 0
        for i in range(total):
            k = i % n
            dur = 1000 * (k + 1) if i < (W + max(1, W)) * n + K * n else 2000 * (k + 1)
            w.writerow({"Kernel_Name": f"void prism::(anonymous namespace)::kern{k}<4>(int)",
                        "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 500
    args = argparse.Namespace(workload=wl.name, pattern="", cus=256, pool_rho=0, dense=False,
                              steps=K, warmup=W, trace_summary=str(path))
    bench.trace_summary(args)
    # with --record-times the graph-replay and eager averages of every kind go
    # to the kernel-times record for this configuration and kernel source
    times = tmp_path / "times.json"
    monkeypatch.setattr(bench, "TIMES_FILE", str(times))
    monkeypatch.setattr(bench, "KERNEL_KINDS", {f"kern{k}": f"kind{k % 2}" for k in range(n)})
    args.record_times = True
    args.int2 = False
    bench.trace_summary(args)
    rec = json.loads(times.read_text())
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()
    e = rec["kernels"]["kind0"][wl.name]
    assert e["dispatches_per_region"] == K * ((n + 1) // 2)
    want_g = np.mean([1.0 * (k + 1) for k in range(0, n, 2)])
    assert abs(e["graph_replay_avg_us"] - want_g) < 1e-3
    assert abs(e["eager_avg_us"] - 2 * want_g) < 1e-3
    assert bench.graph_time_for("kind0", wl.name) == e["graph_replay_avg_us"]
    assert bench.graph_time_for("kind0", "other-workload") is None
    out = capsys.readouterr().out
    row = [l for l in out.splitlines() if "`kern0<4>`" in l][0]
    # graph replay region: 1 us per dispatch; eager region: 2 us
    assert row.startswith("| `kern0<4>` | 1 | 1.00 | 1.00 | 2.00 | 2.00 |")
    # a trace cut short is refused
    with open(path) as f:
        lines = f.read().splitlines()
    path.write_text("\n".join(lines[:-(n + 2)]) + "\n")
    with pytest.raises(SystemExit):
        bench.trace_summary(args)


def test_launch_model_per_workload():
    """The launch counts the benchmark checks its profile rings against, for
    the paths the library takes on 256 compute units: fused kernels at 128K
    planted; anchor and refined layers of the batched and 4 x 128K GQA-8
    workloads in the multi-tile kernels with the rank pool (pools of 4096 and
    16384 entries); with the window pool (pools up to the whole cache) the
    anchor layers select per problem and the refined layers are classified,
    then selected and attended in the multi-tile kernel."""
    import synth
    m = bench.launches_per_step
    p = m(synth.BY_NAME["llama3-8b-128k-planted"], 256)
    assert (p["select"], p["classify"], p["pool_build"], p["attention"]) == (0, 4, 0, 32)
    # rank pool: the anchor layer in the multi-tile kernel on 4 x 128K (six
    # splits per problem), selected per problem on the batched workload (one
    # split per problem would fit)
    for name, na, nr, sel in (("batched-16x8k-64k", 8, 24, 8), ("long-4x128k-gqa8", 10, 70, 0)):
        wl = synth.BY_NAME[name]
        r = m(wl, 256, pool_rho=4)
        assert (r["select"], r["classify"], r["pool_build"]) == (sel, na, 0), (name, r)
        w = m(wl, 256)   # refined layers: classified, then the multi-tile kernel
        assert (w["select"], w["classify"], w["pool_build"]) == (na, na + nr, na), (name, w)
