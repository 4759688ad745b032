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
