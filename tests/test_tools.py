"""Host logic of the measurement tools, on the CPU: bench.py's refusal of
several GPUs and its paired A/B statistics, and bench_profiles.py's reading of
rocprofv3 CSV files (kernel trace runs, counter medians, the traffic scaling)
on small synthetic files whose answers are worked out by hand here."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(args):
    return subprocess.run([sys.executable] + args, cwd=ROOT, capture_output=True, text=True,
                          timeout=120)


def test_bench_refuses_several_gpus():
    r = _run(["bench.py", "--gpus", "2"])
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_ab_stats_verdicts():
    ab = _bench().ab_stats
    rng = np.random.default_rng(7)
    a = 10.0 + rng.normal(0, 0.05, 12)
    same = ab(a, a.copy())
    assert same["ratio_b_over_a"] == 1.0 and same["ci95"] == [1.0, 1.0]
    assert same["verdict"] == "no difference"
    slow = ab(a, a * 1.10 + rng.normal(0, 0.02, 12))
    assert slow["verdict"] == "B slower"
    assert 1.09 < slow["ratio_b_over_a"] < 1.11 and 1.08 < slow["ci95"][0] <= slow["ci95"][1] < 1.12
    fast = ab(a, a * 0.95)
    assert fast["verdict"] == "B faster" and fast["ci95"][1] < 1.0
    # noise of +-2 % around no change: the interval straddles 1
    noisy = ab(a, a * (1.0 + 0.02 * np.array([1, -1] * 6)))
    assert noisy["verdict"] == "no difference"
    assert noisy["ci95"][0] < 1.0 < noisy["ci95"][1]
    # the same seed gives the same interval; the pair count is reported
    assert ab(a, a * 1.01, seed=3) == ab(a, a * 1.01, seed=3)
    assert slow["pairs"] == 12
    with pytest.raises(ValueError):
        ab([1.0, 2.0], [1.0])


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_profile_trace_runs_and_tail(tmp_path):
    # two runs of "attn_kernel" separated by 5 ms of idle time, an unrelated
    # kernel between them; run 0 has durations 10, 12, 11, 13, 20 us
    rows, did, t = [], 0, 1_000_000
    for dur in (10, 12, 11, 13, 20):
        rows.append((did, "attn_kernel", t, t + dur * 1000))
        did += 1
        t += dur * 1000 + 500
    rows.append((did, "other_kernel", t, t + 3000))
    did += 1
    t += 5_000_000
    for dur in (50, 52):
        rows.append((did, "attn_kernel", t, t + dur * 1000))
        did += 1
        t += dur * 1000 + 500
    _write_csv(str(tmp_path / "tr" / "run_kernel_trace.csv"),
               ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    out = tmp_path / "t.md"
    r = _run(["bench_profiles.py", "trace", "--dir", str(tmp_path / "tr"), "--kernel", "attn",
              "--segment", "0", "--tail", "3", "--flops", "1e9", "--title", "T", "--cmd", "c",
              "--out", str(out)])
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    # run 0's last three: 11, 13, 20 us -> mean 14.67, median 13
    assert "runs of 5, 2; run 0 is kept, its last 3" in text
    assert "| count | 3 |" in text and "| mean (us) | 14.67 |" in text
    assert "| median (us) | 13.00 |" in text
    # 1 GFLOP in 13 us
    assert f"| rate at the median | {1e9 / 13e-6 / 1e12:.1f} TFLOP/s |" in text


def _counters(path, kernel_rows):
    rows = []
    for did, name, vals in kernel_rows:
        for cname, v in vals.items():
            rows.append((did, name, cname, v))
    _write_csv(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)


def test_profile_traffic_scaling(tmp_path):
    # the kernel: FETCH_SIZE 100, 300, 200 KiB over three dispatches (median
    # 200, after skipping none), WRITE_SIZE 50 KiB; the 1 GiB copy reads
    # 524288 KiB (so fetch counts are scaled by 2) and writes 1048576 KiB (x1)
    d = tmp_path
    _counters(str(d / "f" / "run_counter_collection.csv"),
              [(i, "attn_kernel", {"FETCH_SIZE": v}) for i, v in enumerate((100.0, 300.0, 200.0))])
    _counters(str(d / "w" / "run_counter_collection.csv"),
              [(i, "attn_kernel", {"WRITE_SIZE": 50.0}) for i in range(3)])
    _counters(str(d / "cf" / "run_counter_collection.csv"),
              [(0, "__amd_rocclr_copyBuffer", {"FETCH_SIZE": 524288.0})])
    _counters(str(d / "cw" / "run_counter_collection.csv"),
              [(0, "__amd_rocclr_copyBuffer", {"WRITE_SIZE": 1048576.0})])
    out, js = d / "t.md", d / "t.json"
    r = _run(["bench_profiles.py", "traffic", "--fetch", str(d / "f"), "--write", str(d / "w"),
              "--copy-fetch", str(d / "cf"), "--copy-write", str(d / "cw"),
              "--algorithmic", "1e5", "--sources", "bench.py", "--kernel", "attn",
              "--title", "T", "--cmd", "c", "--out", str(out), "--json", str(js)])
    assert r.returncode == 0, r.stderr
    rec = json.loads(js.read_text())
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_size_kib_per_dispatch"] == 200.0
    assert rec["hbm_bytes_per_launch"] == 200 * 1024 * 2 + 50 * 1024
    assert len(rec["source_sha256"]) == 64
