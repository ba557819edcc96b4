"""Host-side logic of bench.py (CPU only): the algorithmic byte counts, the
comment-insensitive kernel source hash, and the parsers that turn rocprofv3
CSV output into the committed summaries.  The CSVs here are small synthetic
files in rocprofv3's column layout; nothing runs on a GPU."""

import csv
import json
import os

import pytest

import bench
from fenwick_tree_hierarchical_amd.workloads import WORKLOADS


def test_algorithmic_bytes_16k():
    w = WORKLOADS["train_16k_bf16"]
    c = bench.algorithmic_counts(w, w.B, w.H, w.T, w.dk, w.C, w.L, 2)
    assert c["per_head_token_bytes"] == 4 * 64 * 2 + 4 + 15 * 4 == 576
    assert c["bytes_io"] == 128 * 16384 * 576
    # 256 chunks in 32 groups of 8: 224 chunk nodes, 31 group nodes are read
    assert c["node_bytes_per_bh"] == (224 + 31) * 64 * 64 * 2
    # states: k, v, log_a + 224 chunk nodes + 32 full-group states and totals + 256 chunk totals
    assert c["kernel_bytes"]["chunk_states"] == 128 * (16384 * (2 * 64 * 2 + 4) + 224 * 8192 + 32 * (16384 + 4)
                                                         + 256 * 4)
    assert c["kernel_bytes"]["chunk_output"] == c["bytes_io"] + 128 * ((224 + 31) * 8192 + 256 * 4 + 33 * 8)
    # flops: intra 2 C^2 (2d) per chunk, states 2 C d^2 per chunk, contractions popcount(c) 2 C d^2
    pop = sum(bin(i).count("1") for i in range(256))
    assert c["flops"] == 128 * (256 * 2 * 64 * 64 * 128 + 256 * 2 * 64 * 64 * 64 + pop * 2 * 64 * 64 * 64)


def test_source_hash_ignores_comments_and_whitespace():
    a = "int f(int x) {  // one\n  return x + 1; /* two */ }\n"
    b = "int f(int x){return x+1;}"
    c = "int f(int x){return x+2;}"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    h = bench.kernel_source_hash(read=lambda p: a)
    assert h == bench.kernel_source_hash(read=lambda p: b) != bench.kernel_source_hash(read=lambda p: c)


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_copy_calibration_uses_the_gib_copies_only(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    _counter_csv(str(tmp_path / "f" / "x_counter_collection.csv"),
                 [(copy, "FETCH_SIZE", 524288.0), (copy, "FETCH_SIZE", 131072.0),   # a 1 GiB and a 256 MiB copy
                  (copy, "FETCH_SIZE", 524300.0)])
    _counter_csv(str(tmp_path / "w" / "x_counter_collection.csv"),
                 [(copy, "WRITE_SIZE", 1048576.0), (copy, "WRITE_SIZE", 262144.0), (copy, "WRITE_SIZE", 1048576.0)])
    fk, wk, ff, wf = bench._copy_calibration(str(tmp_path / "f"), str(tmp_path / "w"))
    assert fk == pytest.approx((524288.0 + 524300.0) / 2)
    assert wk == 1048576.0 and wf == 1.0
    assert ff == pytest.approx(1048576.0 / fk)


def test_pmc_profile_scales_each_counter(tmp_path, monkeypatch):
    copy = "__amd_rocclr_copyBuffer"
    out = "void la::fwd_chunk_output<true, 64, 64>(la::FwdArgs)"
    _counter_csv(str(tmp_path / "f" / "a_counter_collection.csv"),
                 [(copy, "FETCH_SIZE", 524288.0), (out, "FETCH_SIZE", 1000.0), (out, "FETCH_SIZE", 1002.0)])
    _counter_csv(str(tmp_path / "w" / "a_counter_collection.csv"),
                 [(copy, "WRITE_SIZE", 1048576.0), (out, "WRITE_SIZE", 500.0), (out, "WRITE_SIZE", 500.0)])
    dst = str(tmp_path / "pmc.json")
    bench.pmc_profile(str(tmp_path / "f"), str(tmp_path / "w"), dst)
    s = json.load(open(dst))
    assert s["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert s["per_launch_kib"]["chunk_output"]["FETCH_SIZE"] == pytest.approx(1001.0)
    assert s["per_kernel_traffic_bytes"]["chunk_output"] == pytest.approx((1001.0 * 2.0 + 500.0) * 1024)
    assert s["kernel_source_hash"] == bench.kernel_source_hash()
    monkeypatch.setattr(bench, "PMC_FILE", dst)
    t, why = bench.pmc_traffic(bench.kernel_source_hash())
    assert why is None and t["chunk_output"] == s["per_kernel_traffic_bytes"]["chunk_output"]
    assert bench.pmc_traffic("0" * 16)[0] is None


def test_trace_summary_groups_by_grid(tmp_path, capsys):
    p = str(tmp_path / "kt_kernel_trace.csv")
    cols = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z",
            "Workgroup_Size_X"]
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for start, end, grid in [(0, 1000, 256), (2000, 4000, 256), (5000, 5500, 1024)]:
            w.writerow({"Kernel_Name": "k", "Start_Timestamp": start, "End_Timestamp": end, "Grid_Size_X": grid,
                        "Grid_Size_Y": 1, "Grid_Size_Z": 1, "Workgroup_Size_X": 256})
    bench.trace_summary(p)
    text = capsys.readouterr().out
    rows = [r for r in text.splitlines() if r.startswith("| `k`")]
    assert len(rows) == 2
    assert "| 256 | 256 | 2 | 1.50 | 1.00 | 2.00 |" in text      # two calls of 1 and 2 us
    assert "| 1024 | 256 | 1 | 0.50 |" in text
