"""Host-side checks of bench.py (no GPU): the one-GPU contract, the traffic
file parsing, and the CPU-baseline leg on a small workload."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_file_matches_current_sources_or_is_ignored():
    import bench

    t = bench.read_traffic()
    assert t is None or t > 0


def test_cpu_baseline_on_the_tiny_workload():
    import bench
    import datagen

    w = datagen.WORKLOADS[1]
    hosts = [datagen.fused_source(w, r) for r in range(w.P)]
    out = bench.cpu_baseline(w, hosts, bench.op_bytes(w), reps=3)
    assert out["kind"] == "oracle" and out["unit"] == "GB/s" and out["value"] > 0
    assert out["cores"] >= 1
    json.dumps(out)
