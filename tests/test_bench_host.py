"""Host-side logic of bench.py (no GPU): the multi-GPU guard, the counted work,
the algorithmic decode bytes, the records' source-hash check, and the pages'
own (ms, TFLOPS) pairs against the counted flops."""
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


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "more_benchmark_l20.txt")


def _page_rows():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        d, case, dtype, nq, nkv, ms, tf = line.split()
        rows.append((d, case, int(nq), int(nkv), ms, tf))
    return rows


def _consistent(flops_of, rows):
    """Every printed (ms, TFLOPS) pair agrees with flops_of(row) once both
    printed numbers are taken as rounded to their last digit."""
    for row in rows:
        d, case, nq, nkv, ms, tf = row
        half_ms = 0.5 * 10.0 ** -len(ms.split(".")[1])
        half_tf = 0.5 * 10.0 ** -(len(tf.split(".")[1]) if "." in tf else 0)
        fl = flops_of(row)
        lo = fl / ((float(ms) + half_ms) * 1e-3) / 1e12
        hi = fl / ((float(ms) - half_ms) * 1e-3) / 1e12
        if not (float(tf) - half_tf <= hi and float(tf) + half_tf >= lo):
            return False
    return True


def test_page_tables_follow_the_counted_flops():
    """The pages' own (ms, TFLOPS) pairs ("FFPA Attention Benchmark", "More
    Benchmark", the L20 forward and backward tables; tests/golden) are
    reproduced by bench.counted_flops: 2 GEMMs forward, 5 backward, causal
    halved, D = 512, with B * H = 32 (8 for the non-aligned rows: the pages
    print neither B nor H, and these are the products their pairs imply).
    Counting the backward as 4 GEMMs, not halving causal, or dropping the
    factor 2 of a GEMM breaks the agreement."""
    rows = _page_rows()
    assert len(rows) == 32

    def bh(case):
        return 8 if case == "non-aligned" else 32

    def ours(row):
        d, case, nq, nkv = row[:4]
        return bench.counted_flops(1, bh(case), nq, nkv, 512, case == "causal", backward=d == "bwd")

    assert _consistent(ours, rows)
    # planted conventions must not fit
    assert not _consistent(lambda r: ours(r) * (0.8 if r[0] == "bwd" else 1.0), rows)
    assert not _consistent(lambda r: ours(r) * (2.0 if r[1] == "causal" else 1.0), rows)
    assert not _consistent(lambda r: ours(r) / 2, rows)


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
