"""bench.py end to end on the GPU: a short run of the default workload prints
one JSON line with every field the benchmark contract names, a roofline
against the 8 TB/s HBM peak, and per-op figures for the four relayouts."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line(gpu):
    import bench

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline", "--no-extras"], capture_output=True, text=True, cwd=ROOT,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert d["metric"] == bench.METRIC
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["dtype"] == "bf16" and d["data"] == "synthetic" and d["vs_baseline"] is None
    assert 0 < d["value"] < 8000 and d["ms_per_step"] > 0
    assert "workload" in d["config"] and d["config"]["bytes_per_step"] == 12710641664
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None or roof["traffic"] > 0
    assert set(d["ops"]) == {"qkv_pack", "qkv_unpack", "attn_split", "head_merge"}
    for op in d["ops"].values():
        assert op["ms"] > 0 and 0 < op["pct_peak"] < 100 and op["launches"] == 6
        assert op["pct_of_d2d_copy"] > 0 and op["pct_of_elementwise_copy"] > 0
    for key in ("qkv", "attn"):
        assert d["copy_elementwise"][key]["gbs"] > 0 and d["copy_d2d"][key]["gbs"] > 0
    assert d["kernel_sources"] == bench.kernel_source_hash()


def test_bench_sections_mid_size(gpu):
    """Every section outside the timed step -- one-chunk windows, the copy
    ceiling, the overlap schedule with each stand-in exchange, head chunks,
    the host cost of a call, head-major layouts and the reference arm -- at
    the mid-size workload.
    Each section checks its own outputs (round trips, windows against the
    whole call, agreement with the direct or token-major results) and makes
    the run exit non-zero otherwise."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "2", "--steps", "3",
                        "--warmup", "1", "--no-cpu-baseline"], capture_output=True, text=True, cwd=ROOT,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads([l for l in r.stdout.splitlines() if l.strip()][-1])
    for key in ("windows", "copy_ceiling", "overlap", "overlap_sdma", "overlap_link_model", "head_chunks",
                "host_cost_us", "head_major", "reference_arm"):
        assert key in d, key
    assert 0 < d["copy_ceiling"]["pct_peak"] < 100
    hc = d["host_cost_us"]
    assert hc["calls"] == 2000 and 0 < hc["c_abi"] < hc["binding"] < 1000
    for op in ("qkv_pack", "qkv_unpack", "attn_split", "head_merge"):
        win = d["windows"][op]
        assert all(win[f"chunk_{c}"]["ms_median"] > 0 for c in range(4))
        assert d["ops"][op]["pct_of_copy_ceiling"] > 0
    ra = d["reference_arm"]
    for op in ("qkv_pack", "qkv_unpack", "attn_split", "attn_split_one_chunk", "head_merge"):
        assert ra[op]["reference_ms"] > 0 and ra[op]["direct_ms"] > 0
    # the allocation screen's factor of two at this workload's sizes (100,663,296 and 33,554,432 B)
    assert ra["qkv_pack"]["direct_peak_bytes"] == 100663296
    assert ra["qkv_pack"]["reference_peak_bytes"] == 2 * 100663296
    assert ra["head_merge"]["direct_peak_bytes"] == 33554432
    assert ra["head_merge"]["reference_peak_bytes"] == 2 * 33554432
    lm = d["overlap_link_model"]
    assert lm["exchange"] == "link" and lm["exchanges_only_ms"] > 0 and lm["overlapped_ms"] > 0
