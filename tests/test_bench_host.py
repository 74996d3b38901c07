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
    out = bench.cpu_baseline(w, hosts, bench.op_bytes(w), reps=3, single_reps=1)
    assert out["kind"] == "oracle" and out["unit"] == "GB/s" and out["value"] > 0
    assert out["cores"] >= 1
    # the chains' peaks: twice the output for the pack and the merge, the
    # factor of the page's allocation screen (24,576 and 8,192 B outputs here)
    nb = bench.op_bytes(w)
    assert out["materialised_peak_bytes"]["qkv_pack"] == nb["qkv_pack"] == 2 * 24576
    assert out["materialised_peak_bytes"]["head_merge"] == nb["head_merge"] == 2 * 8192
    json.dumps(out)


def _counter_csv(path, counter, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, value) in enumerate(rows):
            f.write(f'{i},"{name}",{counter},{value}\n')


def test_pmc_summary_maps_every_kernel_and_calibrates(tmp_path, capsys):
    """Synthetic counter CSVs: FETCH_SIZE reading half the bytes, WRITE_SIZE
    all of them, one kernel per label; the summary must scale both back to
    exactly 1.0x of the algorithmic bytes and name the pack's total."""
    import bench
    import datagen

    w = datagen.WORKLOADS[3]
    nb = bench.op_bytes(w)
    copy_kib = 3 * w.s_local * w.H * w.D * 2 / 1024
    names = {
        ("qkv_pack", "direct"): "void vrl::(anonymous namespace)::relayout_kernel<(vrl::Op)0, 16, true>(vrl::KernelArgs)",
        ("qkv_unpack", "direct"): "void vrl::(anonymous namespace)::relayout_kernel<(vrl::Op)1, 16, true>(vrl::KernelArgs)",
        ("attn_split", "direct"): "void vrl::(anonymous namespace)::relayout_kernel<(vrl::Op)2, 16, true>(vrl::KernelArgs)",
        ("head_merge", "direct"): "void vrl::(anonymous namespace)::relayout_kernel<(vrl::Op)3, 16, true>(vrl::KernelArgs)",
        ("qkv_unpack", "head-run"): "void vrl::(anonymous namespace)::headrun_kernel<(vrl::Op)1, 16>(vrl::KernelArgs)",
        ("head_merge", "head-run"): "void vrl::(anonymous namespace)::headrun_kernel<(vrl::Op)3, 16>(vrl::KernelArgs)",
        ("attn_split", "direct strided-heads"):
            "void vrl::(anonymous namespace)::relayout_kernel<(vrl::Op)2, 16, false>(vrl::KernelArgs)",
    }
    for key, name in names.items():
        assert bench.kernel_label(name) == key
    copy = "void at::native::elementwise_kernel<bitwise_not_kernel>(int, Op)"
    fetch = [(names[(op, kind)], nb[op] / 2 / 1024 / 2) for _, op, kind in bench.PMC_KERNELS]
    write = [(names[(op, kind)], nb[op] / 2 / 1024) for _, op, kind in bench.PMC_KERNELS]
    _counter_csv(str(tmp_path / "f" / "x_counter_collection.csv"), "FETCH_SIZE", fetch + [(copy, copy_kib / 2)])
    _counter_csv(str(tmp_path / "w" / "x_counter_collection.csv"), "WRITE_SIZE", write + [(copy, copy_kib)])
    bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"))
    out = capsys.readouterr().out.splitlines()
    assert out[0] == f"kernel_source_sha256 {bench.kernel_source_hash()}"
    assert out[1] == f"hbm_bytes_per_launch {nb['qkv_pack']}"
    rows = [l for l in out if l.startswith("# ") and l.split()[1] in {"qkv_pack", "qkv_unpack", "attn_split",
                                                                        "head_merge"}]
    assert len(rows) == len(bench.PMC_KERNELS)
    for r in rows:
        assert r.split()[-3:-1] == ["1.0000", "1.0000"], r


def test_trace_summary_labels_workloads_and_windows(tmp_path, capsys):
    """Synthetic kernel trace: whole-tensor launches of the representative and
    P=4 shapes get GB/s from their own algorithmic bytes; a one-chunk window
    launch gets none."""
    import bench

    pack = "void vrl::(anonymous namespace)::relayout_kernel<(vrl::Op)0, 16, true>(vrl::KernelArgs)"
    # grids in work-items: one-wave workgroups of 64 vectors (1 KiB) each
    rows = [(pack, 74479104, 400_000), (pack, 74479104, 400_000),  # representative: 400 us
            (pack, 11907072, 66_000),                              # P=4 whole tensor
            (pack, 18619776, 100_000),                             # one chunk of the representative
            ("__amd_rocclr_copyBuffer", 131072, 50_000)]
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "x_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Grid_Size_X,Start_Timestamp,End_Timestamp\n")
        for name, grid, ns in rows:
            f.write(f'"{name}",{grid},1000,{1000 + ns}\n')
    bench.trace_summary(str(d))
    out = capsys.readouterr().out.splitlines()
    rep = [l for l in out if l.startswith("direct qkv_pack ") and " 74479104 " in l]
    assert len(rep) == 1 and rep[0].split()[-2:] == ["5958", "74.5"], rep   # 2,383,245,312 B / 400 us
    p4 = [l for l in out if l.startswith("direct qkv_pack (P=4)")]
    assert len(p4) == 1 and p4[0].split()[-2:] == ["5773", "72.2"], p4     # 381,026,304 B / 66 us
    win = [l for l in out if l.startswith("direct qkv_pack (window)")]
    assert len(win) == 1 and win[0].split()[-2:] == ["-", "-"]
    assert any(l.startswith("__amd_rocclr_copyBuffer") for l in out)


def test_stats_positions_and_sorted_input():
    """_stats reads median, p10 and p90 by position, so it takes sorted times
    only (the reference arm's two passes are merged and sorted first)."""
    import bench

    ts = [float(i) for i in range(1, 21)]            # 1 .. 20 ms
    s = bench._stats(ts, mean=10.0, nbytes=8_000_000_000)
    assert (s["ms_median"], s["ms_p10"], s["ms_p90"], s["launches"]) == (11.0, 3.0, 19.0, 20)
    assert s["ms_mean_queued"] == 10.0
    assert s["gbs"] == round(8e9 / 11e-3 / 1e9, 1)
    a, b = ts[::2], ts[1::2]                         # two sorted passes
    with pytest.raises(ValueError):
        bench._stats(a + b)
    assert bench._stats(sorted(a + b)) == bench._stats(ts)
