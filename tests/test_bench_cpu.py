"""The bench's host logic, on the CPU: the one-GPU contract, the algorithmic
byte and FLOP counts its roofline divides by, the guard that drops stale
counter data, and the CPU leg's split of a batch over processes."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_counts_follow_their_definitions():
    """Counted from the mask by brute force: the fused launch reads the mask
    and every kept row of q, k and v once, writes every padded output row,
    and writes B + 1 offsets and the longest length (4 bytes each); the
    attention FLOPs are two products of 2 n^2 d per (image, head)."""
    w = W.deit_b_224(0.5)
    st = bench.workload_stats(w)
    R = w.H * w.d * 2
    kept = [int(w.mask[b].sum()) for b in range(w.B)]
    T = sum(kept)
    assert st["T"] == T
    assert st["bytes_fused"] == w.B * w.N + 3 * T * R + w.B * w.N * R + 4 * (w.B + 1) + 4
    assert st["flops"] == sum(2 * 2 * n * n * w.d for n in kept) * w.H
    assert st["bytes_attend"] == 4 * T * R + 4 * (w.B + 1)
    t = W.tiny()
    assert bench.workload_stats(t)["row_bytes"] == t.H * 64 * 4  # fp32 rows


def test_headline_bytes_match_the_recorded_counters():
    """The headline batch's algorithmic bytes are the figure the committed
    counter summary was compared with."""
    d = json.load(open(bench.traffic_file("mixed_b1024")))
    assert bench.workload_stats(W.mixed_peak())["bytes_fused"] == d["algorithmic_bytes_per_launch"]


def test_stale_counters_give_no_traffic(monkeypatch):
    """Counters taken on another version of the kernel are not reported."""
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0000000000000000")
    assert bench.load_traffic("mixed_b1024") is None


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    a, b = tmp_path / "a.hip", tmp_path / "b.hip"
    a.write_text("int f() { return 1; } // one\n/* block */\n")
    b.write_text("int f()  {\n return 1; }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["a.hip"])
    ha = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["b.hip"])
    assert bench.kernel_source_hash() == ha
    b.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash() != ha


@pytest.mark.parametrize("B,parts", [(1024, 16), (2, 16), (4, 3), (7, 7), (1, 1)])
def test_image_ranges_cover_every_image_once(B, parts):
    rng = bench._image_ranges(B, parts)
    covered = np.concatenate([np.arange(b0, b1) for b0, b1 in rng])
    assert np.array_equal(covered, np.arange(B))
    assert len(rng) == min(B, parts)


def test_short_run_summary_takes_the_headlines_first_dispatches(tmp_path, monkeypatch):
    """The short-run trace summary counts the first warm-up + timed
    dispatches of the mixed batch's fused launch shape (later dispatches of
    that shape and other kernels are not the headline's) and compares the
    timed ones with the line's HIP-event figure."""
    import csv
    trace = tmp_path / "trace"
    trace.mkdir()
    (tmp_path / "profiles").mkdir()
    kern = "void rva::" + bench.kernel_label(W.mixed_peak()) + "(rva::AttnParams)"
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Workgroup_Size_Y",
              "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    rows, t = [], 10_000
    for i in range(40):  # 25 headline dispatches, then 15 more of the same shape (1000 us each)
        d = (100 + i) * 1000 if i < 25 else 1_000_000
        rows.append([kern, t, t + d, 256, 1, 1, 6529 * 256, 1, 1])
        rows.append(["void rva::other_kernel()", t + d, t + d + 5000, 256, 1, 1, 256, 1, 1])
        t += d + 10_000
    rows.append([kern, t, t + 7_000_000, 256, 1, 1, 100 * 256, 1, 1])  # another launch shape
    with open(trace / "bench_kernel_trace.csv", "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(fields)
        wr.writerows(rows[::-1])  # order in the file does not matter
    line = tmp_path / "line.json"
    line.write_text("noise\n" + json.dumps({"roofline": {"avg_launch_us": 115.0}}) + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    bench.summarize_short(str(trace), str(line))
    text = (tmp_path / "profiles" / "fused_mixed_b1024_short_run_trace.md").read_text()
    want = sum(100 + i for i in range(5, 25)) / 20  # timed: dispatches 6..25
    assert f"| mean of the 20 timed dispatches (rocprofv3) | {want:.2f} |" in text
    assert "| warm-up 5 | 104.00 |" in text and "| timed 25 | 124.00 |" in text
    assert f"| ratio | {115.0 / want:.4f} |" in text
