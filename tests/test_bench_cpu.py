"""Host-side contract of bench.py: one GPU only, the algorithmic flop count of
the causal score GEMM, and the guard that reports HBM traffic only for the
kernel source it was measured on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_causal_flops_counts_the_triangle():
    # brute force over (t, s <= t) pairs at small sizes
    for L, H, D in ((1, 1, 1), (7, 3, 5), (64, 4, 32)):
        pairs = sum(1 for t in range(L) for s in range(t + 1))
        assert bench.causal_flops(L, H, D) == pairs * H * D * 2
    assert bench.causal_flops(200000, 64, 128) == 327681638400000


def test_traffic_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for_current_kernel() is None          # no file
    f.write_text(json.dumps({"source_sha256": bench.kernel_source_hash(), "traffic_bytes_per_launch": 123.0}))
    assert bench.traffic_for_current_kernel() == 123.0
    f.write_text(json.dumps({"source_sha256": "0" * 64, "traffic_bytes_per_launch": 123.0}))
    assert bench.traffic_for_current_kernel() is None          # kernel changed since the counters
    f.write_text("not json")
    assert bench.traffic_for_current_kernel() is None
