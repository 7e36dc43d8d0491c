"""Host-side logic of bench.py (no GPU): the multi-GPU guard, the counted work,
the algorithmic decode bytes, and the records' source-hash check."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_counted_flops_follow_the_benchmark_convention():
    # forward: 2 GEMMs of 2 B Hq Nq Nkv D; backward: 5; causal halves both
    assert bench.counted_flops(1, 32, 8192, 8192, 512) == 2 ** 42
    assert bench.counted_flops(1, 32, 8192, 8192, 512, causal=True) == 2 ** 41
    assert bench.counted_flops(1, 32, 8192, 8192, 512, backward=True) == 2.5 * 2 ** 42
    assert bench.counted_flops(1, 32, 1024, 8192, 512) == 2 ** 39


def test_decode_bytes_are_k_v_q_o_lse():
    w = W.WORKLOADS["decode"]
    assert bench.decode_bytes(w) == 2 * 16 * 32 * 8192 * 512 * 2 + 2 * 16 * 32 * 512 * 2 + 16 * 32 * 4


def test_source_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    a = tmp_path / "a.hpp"
    b = tmp_path / "b.hpp"
    a.write_text("int x = 1;  // one\n\nint y = 2;\n")
    b.write_text("// header\nint x = 1;\nint y = 2;  // two\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_hash(["a.hpp"]) == bench.kernel_source_hash(["b.hpp"])
    b.write_text("int x = 1;\nint y = 3;\n")
    assert bench.kernel_source_hash(["a.hpp"]) != bench.kernel_source_hash(["b.hpp"])


def test_records_are_dropped_when_the_sources_changed(tmp_path, monkeypatch):
    rec = {"self:f32": {"family": "fwd", "source_sha": "0" * 16, "mfma_util_pct": 1.0}}
    path = tmp_path / "counters.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(path))
    assert bench.recorded_counters("self:f32") is None
    rec["self:f32"]["source_sha"] = bench.kernel_source_hash(bench.COUNTER_SOURCES["fwd"])
    path.write_text(json.dumps(rec))
    assert bench.recorded_counters("self:f32") == {"mfma_util_pct": 1.0}
    assert bench.recorded_counters("missing") is None
