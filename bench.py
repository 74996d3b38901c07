#!/usr/bin/env python3
"""Throughput of the direct sequence<->head relayout on one MI355X.

Workload: the representative 55,413-token shape of the Vflash "Sol-Engine
alignment" page ("What is enabled"): 55,413 tokens padded to 55,414 over
P = 2 ranks (27,707 tokens each), C = 4 chunks, H = 56 heads of 128, BF16,
synthetic N(0,1) values (seed 1, one stream per rank).

A step is one pass of the relayout path for every rank, inputs resident in
HBM: QKV pack, QKV unpack, attention-result split and returned-head merge,
each launched through the C ABI.  The exchanges between them are the
collective's job (RCCL over xGMI on a real multi-GPU run), not the path's;
they run once before timing to fill the receive buffers and are not timed.

Printed: one JSON line with the whole step's effective HBM throughput
(algorithmic bytes: every element read once and written once), per-op
times from HIP events recorded on the launch stream, the roofline of the
dominant kernel (QKV pack) against the 8 TB/s HBM3E peak, copies of the
same bytes for comparison (the runtime's device-to-device copy, torch's
elementwise kernel, and the library's own copy core on a plain contiguous
relayout), sections outside the timed step (one-chunk windows, the overlap
schedule with each stand-in exchange, the other layouts and workloads, the
reference chains), and the CPU oracle timed on the host's cores over one
step of the workload.

Other modes: --mode windows runs only the one-chunk windows (for a kernel
trace of their own); --mode pmc launches each relayout kernel the
representative shape uses, token-major and head-major layouts (rank 0), and
a plain torch copy kernel of known size, for rocprofv3 counter runs;
--mode pmc-sq the kernels of the SQ/TCC counter runs; --pmc-summary,
--sq-summary, --trace-summary and --windows-summary turn the CSVs of such
runs into the summaries kept under profiles/.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QKV-pack / head-merge ms and effective HBM GB/s (% of peak) at 55,413 tokens"
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "relayout_kernels_repr55413_traffic.txt")
# what decides the kernels' memory traffic: device code and launch planning
KERNEL_SOURCES = ["head_relayout_amd/csrc/vrl_kernels.hip", "head_relayout_amd/csrc/vrl_internal.h",
                  "head_relayout_amd/csrc/vrl_plan.cpp"]


def kernel_source_hash() -> str:
    """Hash of the code (comments and whitespace stripped) that decides the
    kernels' memory traffic."""
    import re

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, help="workload id (3 = the representative shape)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip the reference materialisation arm (torch chains, A/direct/A)")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed step: skip the overlap, head-chunk, head-major and "
                         "reference sections (for profiler runs)")
    ap.add_argument("--mode", choices=["bench", "windows", "pmc", "pmc-sq"], default="bench")
    ap.add_argument("--reps", type=int, default=10, help="launches per kernel in --mode pmc")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc output trees (FETCH_SIZE, WRITE_SIZE)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="summarise a rocprofv3 --kernel-trace --stats output tree")
    ap.add_argument("--windows-summary", metavar="DIR",
                    help="summarise the window launches of a kernel trace of --mode windows")
    ap.add_argument("--sq-summary", metavar="DIR",
                    help="summarise a rocprofv3 --pmc output tree of SQ counters per kernel")
    return ap.parse_args()


# ---- device-side setup ---------------------------------------------------------

class Rank:
    """One virtual rank's buffers, all resident in HBM."""

    def __init__(self, w, r, dev, torch, np, datagen, vrl):
        P, C, S_l, H, D, G, S = w.P, w.C, w.s_local, w.H, w.D, w.G, w.S
        self.host = datagen.fused_source(w, r)
        self.fused = torch.from_numpy(self.host.view(np.int16)).to(dev).view(torch.bfloat16)
        self.qkv = [self.fused[:, i * H * D:(i + 1) * H * D].unflatten(1, (H, D)) for i in range(3)]
        n_qkv = vrl.exchange_elems(vrl.VRL_EXCHANGE_QKV, P, C, S_l, H, D)
        n_att = vrl.exchange_elems(vrl.VRL_EXCHANGE_ATTN, P, C, S_l, H, D)
        bf = dict(dtype=torch.bfloat16, device=dev)
        self.packed = torch.empty(n_qkv, **bf)
        self.recv = torch.empty(n_qkv, **bf)
        self.planes = [torch.empty(S, G, D, **bf) for _ in range(3)]
        self.send = torch.empty(n_att, **bf)
        self.back = torch.empty(n_att, **bf)
        self.merged = torch.empty(S_l, H, D, **bf)


def exchange(srcs, dsts, P):
    """All-to-all of P ranks' destination-major wire buffers inside one HBM."""
    for s in range(P):
        for r in range(P):
            dsts[r].view(P, -1)[s].copy_(srcs[s].view(P, -1)[r])


def op_bytes(w) -> dict:
    """Algorithmic bytes per launch (each element read once, written once)."""
    qkv = 2 * 3 * w.s_local * w.H * w.D * 2
    att = 2 * w.s_local * w.H * w.D * 2
    return {"qkv_pack": qkv, "qkv_unpack": qkv, "attn_split": att, "head_merge": att}


def run_bench(args):
    import numpy as np
    import torch

    import datagen
    import head_relayout_amd as vrl

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    w = datagen.WORKLOADS[args.workload]
    P, C = w.P, w.C
    say(f"[bench] workload {w.cid} ({w.name}): generating inputs for {P} ranks")
    ranks = [Rank(w, r, dev, torch, np, datagen, vrl) for r in range(P)]
    torch.cuda.synchronize()

    def pack(rk):
        vrl.qkv_pack(*rk.qkv, rk.packed, P, C)

    def unpack(rk):
        vrl.qkv_unpack(rk.recv, *rk.planes, P, C)

    def split(rk):
        vrl.attn_split(rk.planes[0], rk.send, P, C)

    def merge(rk):
        vrl.head_merge(rk.back, rk.merged, P, C)

    # One full pass with the exchanges, to fill every receive buffer.
    for rk in ranks:
        pack(rk)
    exchange([rk.packed for rk in ranks], [rk.recv for rk in ranks], P)
    for rk in ranks:
        unpack(rk)
        split(rk)
    exchange([rk.send for rk in ranks], [rk.back for rk in ranks], P)
    for rk in ranks:
        merge(rk)
    torch.cuda.synchronize()

    def round_trip_ok() -> bool:
        # merge(exchange(split(unpack(exchange(pack(x))))[Q])) must be x's Q
        return all(torch.equal(rk.merged.view(torch.int16), rk.qkv[0].view(torch.int16))
                   for rk in ranks)

    if not round_trip_ok():
        raise SystemExit("round trip is not bit-exact")

    ops = [("qkv_pack", pack), ("qkv_unpack", unpack), ("attn_split", split), ("head_merge", merge)]
    nbytes = op_bytes(w)
    step_bytes = P * sum(nbytes.values())

    def step(events=None, only=None):
        for name, fn in ops:
            for rk in ranks:
                if events is not None and (only is None or name in only):
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record()
                    fn(rk)
                    b.record()
                    events[name].append((a, b))
                else:
                    fn(rk)

    say(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed region: HIP events only around the pack launches (the
    # roofline kernel).  Every timing event costs the step about 4 us (the
    # queue drains to stamp it), so events around all eight launches would
    # slow the step by some 3 %; the per-op table comes from a second pass
    # that has them.
    say(f"[bench] timing {args.steps} steps (HIP events around the pack launches)")
    pack_events = {name: [] for name, _ in ops}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(pack_events, only=("qkv_pack",))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps

    say(f"[bench] per-op pass: {args.steps} steps with HIP events around every launch")
    events = {name: [] for name, _ in ops}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    ms_per_step_all_events = 1e3 * (time.perf_counter() - t0) / args.steps

    per_op = {}
    for name, _ in ops:
        times = sorted(a.elapsed_time(b) for a, b in events[name])
        mean = sum(times) / len(times)
        gbs = nbytes[name] / (mean * 1e-3) / 1e9
        per_op[name] = {"ms": round(mean, 5), "ms_median": round(times[len(times) // 2], 5),
                        "ms_p10": round(times[len(times) // 10], 5),
                        "ms_p90": round(times[(9 * len(times)) // 10], 5),
                        "ms_min": round(times[0], 5), "bytes": nbytes[name],
                        "gbs": round(gbs, 1), "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 1),
                        "launches": len(times)}

    if not round_trip_ok():
        raise SystemExit("round trip is not bit-exact after timing")

    # Device-to-device copies (hipMemcpyAsync through torch) of the pack's and
    # of the merge's size, for comparison.
    copies = {}
    for name, src in (("qkv", ranks[0].packed), ("attn", ranks[0].send)):
        dst = torch.empty_like(src)
        _warm(torch, lambda _: dst.copy_(src))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / 10
        copies[name] = {"bytes": 2 * src.numel() * 2, "ms": round(ms, 5),
                        "gbs": round(2 * src.numel() * 2 / (ms * 1e-3) / 1e9, 1)}
        del dst
    # A streaming elementwise kernel of torch's (bitwise NOT over the same
    # bytes: one read and one write of each element), median of 20 launches:
    # what a plain vectorised copy-shaped kernel reaches on this part.
    elementwise = {}
    for name, src in (("qkv", ranks[0].packed), ("attn", ranks[0].send)):
        s16 = src.view(torch.int16)
        dst = torch.empty_like(s16)
        _warm(torch, lambda _: torch.bitwise_not(s16, out=dst))
        evs = []
        for _ in range(20):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            torch.bitwise_not(s16, out=dst)
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in evs)[10]
        elementwise[name] = {"kernel": "torch.bitwise_not (int16)", "bytes": 2 * src.numel() * 2,
                             "ms_median": round(ms, 5),
                             "gbs": round(2 * src.numel() * 2 / (ms * 1e-3) / 1e9, 1)}
        del dst
    say("[bench] copy ceiling: the library's copy core on a plain contiguous relayout")
    ceiling = copy_ceiling(torch, vrl, w)
    for name in per_op:
        key = "qkv" if name in ("qkv_pack", "qkv_unpack") else "attn"
        per_op[name]["pct_of_d2d_copy"] = round(100 * per_op[name]["gbs"] / copies[key]["gbs"], 1)
        med_gbs = nbytes[name] / (per_op[name]["ms_median"] * 1e-3) / 1e9   # medians on both sides
        per_op[name]["pct_of_elementwise_copy"] = round(100 * med_gbs / elementwise[key]["gbs"], 1)
        per_op[name]["pct_of_copy_ceiling"] = round(100 * med_gbs / ceiling["gbs"], 1)

    # the dominant kernel's mean launch duration, from the timed region's events
    dominant = "qkv_pack"
    dom_times = [a.elapsed_time(b) for a, b in pack_events[dominant]]
    achieved = round(nbytes[dominant] / (sum(dom_times) / len(dom_times) * 1e-3) / 1e9, 1)
    roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": read_traffic(),
                "kernel": "qkv_pack (relayout_kernel<Pack, 16 B, contiguous>)",
                "bytes_per_launch": nbytes[dominant], "launches": len(dom_times)}

    result = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_events_on_every_launch": round(ms_per_step_all_events, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.total_tokens} tokens padded to {w.S}, P={P} ranks x "
                               f"{w.s_local} tokens, C={C}, H={w.H}, D={w.D}",
                   "P": P, "C": C, "s_local": w.s_local, "H": w.H, "D": w.D,
                   "step": "qkv_pack + qkv_unpack + attn_split + head_merge for each rank",
                   "bytes_per_step": step_bytes},
        "ops": per_op,
        "roofline": roofline,
        "copy_d2d": copies,
        "copy_elementwise": elementwise,
        "copy_ceiling": ceiling,
        "verified": "round trip bit-exact before and after timing",
        "kernel_sources": kernel_source_hash(),
    }
    say("[bench] the step captured in a HIP graph")
    result["graph_replay"] = graph_replay(torch, ops, ranks, step_bytes, args.steps)
    if not round_trip_ok():
        raise SystemExit("round trip is not bit-exact after graph replays")
    if not args.no_extras:
        say("[bench] one-chunk windows")
        result["windows"] = chunk_windows(torch, vrl, w, ranks)
        say("[bench] four-chunk overlap schedule")
        kernels_ms = round(P * sum(per_op[n]["ms"] for n in per_op), 4)
        result["overlap"] = overlap_schedule(torch, w, ranks, kernels_ms=kernels_ms)
        result["overlap_sdma"] = overlap_schedule(torch, w, ranks, engine="sdma", kernels_ms=kernels_ms)
        say("[bench] four-chunk overlap schedule, link-paced exchange")
        result["overlap_link_model"] = overlap_schedule(torch, w, ranks, engine="link", kernels_ms=kernels_ms)
        say("[bench] head-chunked layout")
        result["head_chunks"] = head_chunk_layout(torch, vrl, w, ranks)
        say("[bench] host cost of one call")
        result["host_cost_us"] = host_cost(torch, vrl)
        say("[bench] head-major (BHTD) attention side")
        result["head_major"] = head_major_layouts(torch, vrl, w, ranks[0])
        if w.cid == 3:
            say("[bench] head-major layouts with narrow heads")
            result["head_major_narrow"] = head_major_narrow(torch, np, datagen, vrl, dev)
        if w.cid == 3:
            say("[bench] padded source rows (row stride 21,568)")
            result["strided_rows"] = strided_rows(torch, np, datagen, vrl, dev)
            say("[bench] mid-size and P=4 workloads (buffer rotation past the Infinity Cache)")
            result["smaller_workloads"] = smaller_workloads(torch, np, datagen, vrl, dev)
    if not args.no_reference and not args.no_extras:
        say("[bench] reference materialisation arm (A/direct/A)")
        result["reference_arm"] = reference_arm(torch, vrl, w, ranks)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, [rk.host for rk in ranks], nbytes)
    print(json.dumps(result), flush=True)


# ---- timing helpers -------------------------------------------------------------

# Warm-up before every timed series, in ms of calls.  After the GPU has sat
# idle (host-side input generation between sections) the LDS transpose runs
# at about 76 % for a few calls, dips to 67-70 % around the tenth and settles
# back near 75 % after some 25 calls (10 ms), while the clock finds its level;
# the copy kernels barely move.  A fixed count of three warm-up calls timed
# that dip instead of the steady rate.
WARM_MS = 50.0


def _warm(torch, fn, sets=(None,), ms=WARM_MS):
    """fn(set) called, cycling through `sets`, until at least `ms` ms of wall
    time have passed with the stream drained (and at least three calls)."""
    t0, n = time.perf_counter(), 0
    while n < 3 or 1e3 * (time.perf_counter() - t0) < ms:
        for _ in range(4):
            out = fn(sets[n % len(sets)])
            del out
            n += 1
        torch.cuda.synchronize()


def _queued(torch, fn, sets, reps):
    """fn(set) called `reps` times, cycling through `sets`, queued back to
    back on the current stream with no host synchronisation in between, in
    two passes: one with HIP events around every call (sorted per-call times)
    and one with events only around the whole queue (mean per call, the
    queue's throughput without the per-call events).  Times in ms, after a
    warm-up of WARM_MS.  Whatever fn returns is dropped as soon as it is
    queued, so a chain's own allocations are recycled by torch's allocator."""
    _warm(torch, fn, sets)
    pairs = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        out = fn(sets[i % len(sets)])
        e1.record()
        del out
        pairs.append((e0, e1))
    q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    q0.record()
    for i in range(reps):
        out = fn(sets[i % len(sets)])
        del out
    q1.record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in pairs), q0.elapsed_time(q1) / reps


def _stats(ts, mean=None, nbytes=None) -> dict:
    """Median, p10, p90 and count of sorted per-call times `ts` (ms), with the
    queue mean and the rate for `nbytes` when given."""
    if any(a > b for a, b in zip(ts, ts[1:])):
        raise ValueError("_stats needs sorted times")
    n = len(ts)
    out = {"ms_median": round(ts[n // 2], 5), "ms_p10": round(ts[n // 10], 5),
           "ms_p90": round(ts[(9 * n) // 10], 5), "launches": n}
    if mean is not None:
        out["ms_mean_queued"] = round(mean, 5)
    if nbytes is not None:
        gbs = nbytes / (ts[n // 2] * 1e-3) / 1e9
        out.update({"bytes": nbytes, "gbs": round(gbs, 1), "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 1)})
    return out


def _sets_for(nbytes: int, have: int) -> int:
    """Buffer sets to rotate so that k x bytes per launch >= 1 GiB (the 256 MB
    Infinity Cache then holds none of a launch's inputs), at most `have`."""
    return max(1, min(have, -(-(1 << 30) // nbytes)))


# ---- the reference materialisation chains on the GPU (comparison arm) ----------

def reference_arm(torch, vrl, w, ranks, reps=16):
    """A/direct/A of the reference chains (harness/reference_chains.py)
    against the direct relayouts, and their incremental peak allocations.
    Each arm's calls are queued back to back, so the GPU times hold neither
    the binding's host cost nor idle gaps; inputs rotate over enough buffers
    that every call reads from HBM; the direct calls write into outputs
    allocated beforehand, while the chains allocate theirs as they go (that
    is what they do; torch's allocator recycles them, no device allocation
    happens in the timed region)."""
    from harness import reference_chains as rc

    P, C, S_l, H, D, G, S = w.P, w.C, w.s_local, w.H, w.D, w.G, w.S
    bf = dict(dtype=torch.bfloat16, device=ranks[0].fused.device)
    T0 = vrl.chunk_offset(1, P, C, S_l, H, D)
    nb = op_bytes(w)
    packed_out = torch.empty_like(ranks[0].packed)
    planes_out = [torch.empty(S, G, D, **bf) for _ in range(3)]
    send_out = torch.empty_like(ranks[0].send)
    merged_out = torch.empty(S_l, H, D, **bf)
    qkv_sets = [rk.qkv for rk in ranks]
    recv_sets = [rk.recv for rk in ranks]
    o_sets = [p for rk in ranks for p in rk.planes]
    ret_sets = [t for rk in ranks for t in (rk.back, rk.send)]
    one_chunk = 2 * P * T0 * G * D * 2
    arms = {
        "qkv_pack": (qkv_sets, nb["qkv_pack"], lambda x: rc.ref_pack(torch, *x, P, C),
                     lambda x: vrl.qkv_pack(*x, packed_out, P, C), lambda: packed_out),
        "qkv_unpack": (recv_sets, nb["qkv_unpack"], lambda x: rc.ref_unpack(torch, x, P, C, S_l, G, D),
                       lambda x: vrl.qkv_unpack(x, *planes_out, P, C), lambda: planes_out),
        "attn_split": (o_sets, nb["attn_split"], lambda x: rc.ref_split(torch, x, P, C),
                       lambda x: vrl.attn_split(x, send_out, P, C), lambda: send_out),
        "attn_split_one_chunk": (o_sets, one_chunk, lambda x: rc.ref_split(torch, x, P, C, 0, 1),
                                 lambda x: vrl.attn_split(x, send_out, P, C, 0, 1),
                                 lambda: send_out.view(P, S_l * G * D)[:, :T0 * G * D]),
        "head_merge": (ret_sets, nb["head_merge"], lambda x: rc.ref_merge(torch, x, P, S_l, G, D),
                       lambda x: vrl.head_merge(x, merged_out, P, C), lambda: merged_out),
    }
    res = {}
    for name, (sets, nbytes, ref_fn, dir_fn, dir_out) in arms.items():
        k = _sets_for(nbytes, len(sets))
        sets = sets[:k]
        # bit-exact agreement of the two arms on the first set
        a = ref_fn(sets[0])
        dir_fn(sets[0])
        b = dir_out()
        a = a if isinstance(a, list) else [a]
        b = b if isinstance(b, list) else [b]
        for x, y in zip(a, b):
            if not torch.equal(x.reshape(-1).view(torch.int16), y.reshape(-1).view(torch.int16)):
                raise SystemExit(f"reference and direct {name} differ")
        del a, b
        ra, ra_mean = _queued(torch, ref_fn, sets, reps)
        dm, dm_mean = _queued(torch, dir_fn, sets, reps)
        rb, rb_mean = _queued(torch, ref_fn, sets, reps)
        ref_med = (ra[len(ra) // 2] + rb[len(rb) // 2]) / 2
        entry = {"reference": _stats(sorted(ra + rb), (ra_mean + rb_mean) / 2), "direct": _stats(dm, dm_mean),
                 "reference_ms": round(ref_med, 5), "direct_ms": round(dm[len(dm) // 2], 5),
                 "speedup": round(ref_med / dm[len(dm) // 2], 3), "bytes": nbytes, "buffer_sets": k}
        if name == "attn_split_one_chunk":
            entry["output_bytes"] = P * T0 * G * D * 2
            entry["reference_peak_bytes"] = rc.peak_bytes(torch, lambda: ref_fn(sets[0]))
        res[name] = entry
    # incremental peak allocations: each arm with an output of its own
    rk = ranks[0]

    def d_pack():
        out = torch.empty(rk.packed.numel(), **bf)
        vrl.qkv_pack(*rk.qkv, out, P, C)
        return out

    def d_unpack():
        outs = [torch.empty(S, G, D, **bf) for _ in range(3)]
        vrl.qkv_unpack(rk.recv, *outs, P, C)
        return outs

    def d_split():
        out = torch.empty(rk.send.numel(), **bf)
        vrl.attn_split(rk.planes[0], out, P, C)
        return out

    def d_merge():
        out = torch.empty(S_l, H, D, **bf)
        vrl.head_merge(rk.back, out, P, C)
        return out

    for name, ref_fn, dir_fn in (
            ("qkv_pack", lambda: rc.ref_pack(torch, *rk.qkv, P, C), d_pack),
            ("qkv_unpack", lambda: rc.ref_unpack(torch, rk.recv, P, C, S_l, G, D), d_unpack),
            ("attn_split", lambda: rc.ref_split(torch, rk.planes[0], P, C), d_split),
            ("head_merge", lambda: rc.ref_merge(torch, rk.back, P, S_l, G, D), d_merge)):
        res[name]["reference_peak_bytes"] = rc.peak_bytes(torch, ref_fn)
        res[name]["direct_peak_bytes"] = rc.peak_bytes(torch, dir_fn)
    del packed_out, planes_out, send_out, merged_out
    return res


def chunk_windows(torch, vrl, w, ranks, reps=24):
    """One-chunk windows [c, c+1) of the four relayouts, c = 0 .. C-1 (token
    chunks), nothing else running: per-launch HIP events of calls queued
    back to back over k buffer sets (k x window bytes >= 1 GiB, so every
    launch reads from HBM), and the mean per launch of the whole queue.  The
    windows composed over every chunk are checked equal to the whole call."""
    P, C, S_l, H, D, G, S = w.P, w.C, w.s_local, w.H, w.D, w.G, w.S
    bf = dict(dtype=torch.bfloat16, device=ranks[0].fused.device)
    off = [vrl.chunk_offset(c, P, C, S_l, H, D) for c in range(C + 1)]
    n_att = S_l * H * D
    res = {}
    for name in ("qkv_pack", "qkv_unpack", "attn_split", "head_merge"):
        planes3 = name in ("qkv_pack", "qkv_unpack")
        win_bytes = [2 * (3 if planes3 else 1) * (off[c + 1] - off[c]) * H * D * 2 for c in range(C)]
        k = _sets_for(min(win_bytes), 6)
        if name == "qkv_pack":
            ins = [rk.qkv for rk in ranks]
            outs = [torch.empty_like(ranks[0].packed) for _ in range(k)]
            call = lambda i, o, cb, ce: vrl.qkv_pack(*i, o, P, C, cb, ce)  # noqa: E731
        elif name == "qkv_unpack":
            ins = [rk.recv for rk in ranks]
            outs = [[torch.empty(S, G, D, **bf) for _ in range(3)] for _ in range(k)]
            call = lambda i, o, cb, ce: vrl.qkv_unpack(i, *o, P, C, cb, ce)  # noqa: E731
        elif name == "attn_split":
            ins = [p for rk in ranks for p in rk.planes]
            outs = [torch.empty(n_att, **bf) for _ in range(k)]
            call = lambda i, o, cb, ce: vrl.attn_split(i, o, P, C, cb, ce)  # noqa: E731
        else:
            ins = [t for rk in ranks for t in (rk.back, rk.send, rk.packed[:n_att])]
            outs = [torch.empty(S_l, H, D, **bf) for _ in range(k)]
            call = lambda i, o, cb, ce: vrl.head_merge(i, o, P, C, cb, ce)  # noqa: E731
        sets = [(ins[j % len(ins)], outs[j]) for j in range(k)]
        entry = {"buffer_sets": k}
        for c in range(C):
            for st in sets:
                call(*st, c, c + 1)
            ts, mean = _queued(torch, lambda st, c=c: call(*st, c, c + 1), sets, reps)
            entry[f"chunk_{c}"] = _stats(ts, mean, win_bytes[c])
        # composed windows == whole call (set 0's output holds every window now)
        whole = (torch.empty_like(outs[0]) if not isinstance(outs[0], list)
                 else [torch.empty_like(t) for t in outs[0]])
        call(sets[0][0], whole, 0, C)
        torch.cuda.synchronize()
        a = outs[0] if isinstance(outs[0], list) else [outs[0]]
        b = whole if isinstance(whole, list) else [whole]
        if not all(torch.equal(x.view(torch.int16), y.view(torch.int16)) for x, y in zip(a, b)):
            raise SystemExit(f"{name}: the one-chunk windows composed differ from the whole call")
        res[name] = entry
        del outs, sets, whole, a, b
    return res


def copy_ceiling(torch, vrl, w, reps=20):
    """The library's direct kernel on a relayout that is a plain contiguous
    copy: a QKV pack with P = 1 and C = 1 from three dense [S_l][H][D]
    tensors (each plane one contiguous block), moving the pack's bytes.  What
    the same copy core reaches without any index swap."""
    S_l, H, D = w.s_local, w.H, w.D
    dev = torch.device("cuda:0")
    qkv = [torch.empty(S_l, H, D, dtype=torch.int16, device=dev).random_(-30000, 30000).view(torch.bfloat16)
           for _ in range(3)]
    out = torch.empty(3 * S_l * H * D, dtype=torch.bfloat16, device=dev)
    fn = lambda _: vrl.qkv_pack(*qkv, out, 1, 1)  # noqa: E731
    ts, mean = _queued(torch, fn, [None], reps)
    if not torch.equal(out.view(torch.int16), torch.cat([t.reshape(-1) for t in qkv]).view(torch.int16)):
        raise SystemExit("copy ceiling: the P = 1 pack is not a plain copy")
    entry = _stats(ts, mean, op_bytes(w)["qkv_pack"])
    entry["kernel"] = "relayout_kernel<Pack, 16 B, contiguous> with P = 1, C = 1 (three contiguous copies)"
    del qkv, out
    return entry


def graph_replay(torch, ops, ranks, step_bytes, steps):
    """The step (all four relayouts for every rank) captured once in a HIP
    graph and replayed: the same kernels and arguments without per-launch
    host work between them."""
    def step():
        for _, fn in ops:
            for rk in ranks:
                fn(rk)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / steps
    del g
    return {"ms_per_step": round(ms, 4), "gbs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
            "steps": steps}


def overlap_schedule(torch, w, ranks, reps=10, engine="kernel", kernels_ms=None):
    """The whole layer, exchanges included: the exchanges alone, the serial
    schedule (each stage over all chunks, one after the other) and the
    four-chunk overlap schedule (per-chunk stages, exchanges on a second
    stream, event-ordered ready waits).  engine picks the stand-in exchange
    (harness/ulysses.py): copy kernels or SDMA copies inside the one HBM,
    which compete with the relayouts for bandwidth, or link-paced copies,
    which take each block between two ranks at one xGMI link's rate and so
    cost the HBM only what the links would carry.  exposed_* = schedule time
    minus the exchanges alone: the relayout time the schedule leaves
    uncovered.  kernels_ms: the layer's relayouts alone (every rank's four
    calls, from the timed step)."""
    from harness.ulysses import Layer, run_exchanges, run_overlapped, run_serial

    layer = Layer(w.P, w.C, w.s_local, w.H, w.D, engine)
    comm = torch.cuda.Stream()
    out = {"exchange": engine}
    if engine == "link":
        out["link_gbs"] = layer.link_gbs
    for name, fn in (("exchanges_only", lambda: run_exchanges(layer, ranks)),
                     ("serial", lambda: run_serial(layer, ranks)),
                     ("overlapped", lambda: run_overlapped(layer, ranks, comm))):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        out[name + "_ms"] = round(1e3 * (time.perf_counter() - t0) / reps, 4)
    out["exposed_serial_ms"] = round(out["serial_ms"] - out["exchanges_only_ms"], 4)
    out["exposed_overlapped_ms"] = round(out["overlapped_ms"] - out["exchanges_only_ms"], 4)
    if kernels_ms is not None:
        out["kernels_ms"] = kernels_ms
    waits = {}
    run_overlapped(layer, ranks, comm, waits=waits)
    torch.cuda.synchronize()
    for kind, pairs in waits.items():
        out[kind + "_ready_wait_ms"] = round(sum(a.elapsed_time(b) for a, b in pairs), 4)
    if not all(torch.equal(rk.merged.view(torch.int16), rk.qkv[0].view(torch.int16)) for rk in ranks):
        raise SystemExit(f"overlap schedule ({engine} exchange): round trip is not bit-exact")
    out["chunks"] = w.C
    return out


def _median_ms(torch, fn, reps=10):
    _warm(torch, lambda _: fn())
    pairs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in pairs)[reps // 2]


def head_chunk_layout(torch, vrl, w, ranks):
    """The four relayouts with the chunks splitting head groups (chunk_heads),
    on the same tensors, with a real exchange between the ranks' wire buffers;
    the round trip is checked bit-exact."""
    P, C, S_l, H, D, G, S = w.P, w.C, w.s_local, w.H, w.D, w.G, w.S
    hc = dict(chunk_heads=True)
    bf = dict(dtype=torch.bfloat16, device=ranks[0].fused.device)
    packed = [torch.empty_like(rk.packed) for rk in ranks]
    recv = [torch.empty_like(rk.packed) for rk in ranks]
    planes = [[torch.empty(S, G, D, **bf) for _ in range(3)] for _ in ranks]
    send = [torch.empty_like(rk.send) for rk in ranks]
    back = [torch.empty_like(rk.send) for rk in ranks]
    merged = [torch.empty(S_l, H, D, **bf) for _ in ranks]
    for r, rk in enumerate(ranks):
        vrl.qkv_pack(*rk.qkv, packed[r], P, C, **hc)
    exchange(packed, recv, P)
    for r in range(P):
        vrl.qkv_unpack(recv[r], *planes[r], P, C, **hc)
        vrl.attn_split(planes[r][0], send[r], P, C, **hc)
    exchange(send, back, P)
    for r in range(P):
        vrl.head_merge(back[r], merged[r], P, C, **hc)
    torch.cuda.synchronize()
    for r, rk in enumerate(ranks):
        if not torch.equal(merged[r].view(torch.int16), rk.qkv[0].view(torch.int16)):
            raise SystemExit("head-chunked round trip is not bit-exact")
        if not all(torch.equal(planes[r][q].view(torch.int16), rk.planes[q].view(torch.int16))
                   for q in range(3)):
            raise SystemExit("head-chunked unpack differs from token-chunked unpack")
    nb = op_bytes(w)
    out = {}
    for name, fn in (("qkv_pack", lambda: vrl.qkv_pack(*ranks[0].qkv, packed[0], P, C, **hc)),
                     ("qkv_unpack", lambda: vrl.qkv_unpack(recv[0], *planes[0], P, C, **hc)),
                     ("attn_split", lambda: vrl.attn_split(planes[0][0], send[0], P, C, **hc)),
                     ("head_merge", lambda: vrl.head_merge(back[0], merged[0], P, C, **hc))):
        ms = _median_ms(torch, fn)
        gbs = nb[name] / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 5), "gbs": round(gbs, 1), "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 1)}
    # one chunk window, rotating over every plane of every rank (and as many
    # outputs) so that each launch reads from HBM
    one = 2 * S * (G // C) * D * 2
    sets = [(planes[r][q], send[r]) for r in range(P) for q in range(3)][:_sets_for(one, 3 * P)]
    for o, sd in sets:
        vrl.attn_split(o, sd, P, C, 0, 1, **hc)
    ts, mean = _queued(torch, lambda st: vrl.attn_split(st[0], st[1], P, C, 0, 1, **hc), sets, 24)
    out["attn_split_one_chunk"] = _stats(ts, mean, one)
    out["attn_split_one_chunk"]["output_bytes"] = S * (G // C) * D * 2
    return out


def host_cost(torch, vrl, calls=2000):
    """Host time to enqueue one call, in microseconds: a one-chunk split of
    a tiny attention output (two ranks of 64 tokens, 2 x 4 heads of 16), so
    that the GPU stays ahead of the host and the launch queue never fills.
    Through the C ABI by ctypes with the arguments built once (validation,
    the device, stream and pointer-attribute queries and the launch), and
    through the torch binding (which also builds the arguments from the
    tensors).  No synchronisation inside the timed loops."""
    import ctypes

    from head_relayout_amd import _lib

    P, C, S_l, H, D = 2, 4, 64, 8, 16
    G, S = H // P, P * S_l
    dev = torch.device("cuda:0")
    o = torch.empty(S, G, D, dtype=torch.int16, device=dev).random_(-30000, 30000).view(torch.bfloat16)
    send = torch.zeros(S * G * D, dtype=torch.bfloat16, device=dev)
    lib = _lib.lib()
    dims = _lib.Dims(P, C, S_l, H, D, 0)
    view = _lib.View(o.data_ptr(), G * D, D)
    stream = torch.cuda.current_stream().cuda_stream

    def c_abi():
        if lib.vrl_attn_split(ctypes.byref(dims), ctypes.byref(view), send.data_ptr(), 0, 1, stream) != 0:
            raise SystemExit("host cost: the C-ABI call failed")

    def binding():
        vrl.attn_split(o, send, P, C, 0, 1)

    out = {"calls": calls}
    for name, fn in (("c_abi", c_abi), ("binding", binding)):
        for _ in range(50):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(calls):
            fn()
        t1 = time.perf_counter()
        torch.cuda.synchronize()
        out[name] = round(1e6 * (t1 - t0) / calls, 2)
    if not torch.equal(send.view(torch.int16)[:S_l // C * G * D], o.view(torch.int16).reshape(-1)[:S_l // C * G * D]):
        raise SystemExit("host cost: the one-chunk split wrote the wrong bytes")
    return out


def head_major_layouts(torch, vrl, w, rk):
    """Unpack into, and split from, attention-side tensors stored head-major
    ([G][S][D], viewed as [S][G][D]), and merge into a head-major output
    ([H][S_l][D], viewed as [S_l][H][D]); checked against the token-major
    results."""
    P, C, S_l, H, D, G, S = w.P, w.C, w.s_local, w.H, w.D, w.G, w.S
    bf = dict(dtype=torch.bfloat16, device=rk.fused.device)
    hm = [torch.empty(G, S, D, **bf) for _ in range(3)]
    views = [t.transpose(0, 1) for t in hm]
    send = torch.empty_like(rk.send)
    merged = torch.empty(H, S_l, D, **bf)
    nb = op_bytes(w)
    out = {}
    for name, fn, nbytes in (
            ("qkv_unpack", lambda: vrl.qkv_unpack(rk.recv, *views, P, C), nb["qkv_unpack"]),
            ("attn_split", lambda: vrl.attn_split(views[0], send, P, C), nb["attn_split"]),
            ("head_merge", lambda: vrl.head_merge(rk.back, merged.transpose(0, 1), P, C), nb["head_merge"])):
        ms = _median_ms(torch, fn)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 5), "gbs": round(gbs, 1), "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 1)}
    for q in range(3):
        if not torch.equal(views[q].reshape(-1, D).view(torch.int16).contiguous(),
                           rk.planes[q].reshape(-1, D).view(torch.int16)):
            raise SystemExit("head-major unpack differs from token-major unpack")
    if not torch.equal(send.view(torch.int16), rk.send.view(torch.int16)):
        raise SystemExit("split from head-major O differs from split from token-major O")
    if not torch.equal(merged.transpose(0, 1).contiguous().view(torch.int16), rk.merged.view(torch.int16)):
        raise SystemExit("merge into a head-major output differs from the token-major merge")
    return out


def head_major_narrow(torch, np, datagen, vrl, dev, dims=(16, 32)):
    """Head-major attention side and merge output with narrow heads (16 and
    32 elements: head rows below one cache line, the LDS transpose), 56 heads,
    the token count per rank scaled so every op moves the representative
    shape's bytes; checked against the token-major results."""
    base = datagen.WORKLOADS[3]
    out = {}
    for D in dims:
        w = datagen.Workload(0, f"head_dim {D}", P=base.P, C=base.C, s_local=base.s_local * base.D // D,
                             H=base.H, D=D, total_tokens=base.P * base.s_local * base.D // D, seed=base.seed)
        P, C, S_l, H, G, S = w.P, w.C, w.s_local, w.H, w.G, w.S
        bf = dict(dtype=torch.bfloat16, device=dev)
        rk = Rank(w, 0, dev, torch, np, datagen, vrl)
        vrl.qkv_pack(*rk.qkv, rk.packed, P, C)
        vrl.qkv_unpack(rk.packed, *rk.planes, P, C)          # token-major reference results
        vrl.attn_split(rk.planes[0], rk.send, P, C)
        vrl.head_merge(rk.send, rk.merged, P, C)
        hm = [torch.empty(G, S, D, **bf) for _ in range(3)]
        views = [t.transpose(0, 1) for t in hm]
        send = torch.empty_like(rk.send)
        merged = torch.empty(H, S_l, D, **bf)
        nb = op_bytes(w)
        res = {"s_local": S_l, "D": D}
        for name, fn in (("qkv_unpack", lambda: vrl.qkv_unpack(rk.packed, *views, P, C)),
                         ("attn_split", lambda: vrl.attn_split(views[0], send, P, C)),
                         ("head_merge", lambda: vrl.head_merge(rk.send, merged.transpose(0, 1), P, C))):
            ms = _median_ms(torch, fn)
            gbs = nb[name] / (ms * 1e-3) / 1e9
            res[name] = {"ms": round(ms, 5), "gbs": round(gbs, 1), "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 1)}
        torch.cuda.synchronize()
        same = all(torch.equal(views[q].contiguous().view(torch.int16), rk.planes[q].view(torch.int16))
                   for q in range(3))
        same = same and torch.equal(send.view(torch.int16), rk.send.view(torch.int16))
        same = same and torch.equal(merged.transpose(0, 1).contiguous().view(torch.int16),
                                    rk.merged.view(torch.int16))
        if not same:
            raise SystemExit(f"head-major layouts at head_dim {D} differ from the token-major results")
        out[f"head_dim_{D}"] = res
        del rk, hm, views, send, merged
    return out


def strided_rows(torch, np, datagen, vrl, dev):
    """The representative shape with every token row of the fused QKV source
    padded to 21,568 elements (Q/K/V at column offsets 0 / 7,168 / 14,336, 64
    sentinel pad columns): pack from those rows, and merge both into a dense
    [S_l][H][D] output and into rows of the same padded stride.  The round
    trip must return Q bit for bit and leave the pad columns untouched."""
    w = datagen.WORKLOADS[4]
    P, C, S_l, H, D = w.P, w.C, w.s_local, w.H, w.D
    ranks = [Rank(w, r, dev, torch, np, datagen, vrl) for r in range(P)]
    for rk in ranks:
        vrl.qkv_pack(*rk.qkv, rk.packed, P, C)
    exchange([rk.packed for rk in ranks], [rk.recv for rk in ranks], P)
    for rk in ranks:
        vrl.qkv_unpack(rk.recv, *rk.planes, P, C)
        vrl.attn_split(rk.planes[0], rk.send, P, C)
    exchange([rk.send for rk in ranks], [rk.back for rk in ranks], P)
    rk = ranks[0]
    row = rk.fused.shape[1]
    padded = torch.full((S_l, row), datagen.PAD_SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    padded_view = padded[:, :H * D].unflatten(1, (H, D))
    nb = op_bytes(w)
    out = {"row_stride_elems": row}
    for name, fn, nbytes in (
            ("qkv_pack", lambda: vrl.qkv_pack(*rk.qkv, rk.packed, P, C), nb["qkv_pack"]),
            ("head_merge", lambda: vrl.head_merge(rk.back, rk.merged, P, C), nb["head_merge"]),
            ("head_merge_padded_rows", lambda: vrl.head_merge(rk.back, padded_view, P, C),
             nb["head_merge"])):
        ms = _median_ms(torch, fn)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 5), "gbs": round(gbs, 1), "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 1)}
    torch.cuda.synchronize()
    q = rk.qkv[0].reshape(S_l, H * D).view(torch.int16)
    if not (torch.equal(rk.merged.view(S_l, H * D).view(torch.int16), q)
            and torch.equal(padded[:, :H * D].view(torch.int16), q)):
        raise SystemExit("padded-row round trip is not bit-exact")
    if not bool((padded[:, H * D:].view(torch.int16) == datagen.PAD_SENTINEL).all()):
        raise SystemExit("merge into padded rows touched the pad columns")
    return out


def shard_workloads(datagen):
    """One rank's share of the representative 55,413-token sequence over 4
    and 8 ranks (55,416 tokens after padding; 56 heads of 128, four token
    chunks): the shapes each GPU of a four- or eight-GPU run would relayout."""
    base = datagen.WORKLOADS[3]
    return [datagen.Workload(0, f"representative sequence over P={P}", P=P, C=base.C,
                             s_local=-(-base.total_tokens // P), H=base.H, D=base.D,
                             total_tokens=base.total_tokens, seed=base.seed) for P in (4, 8)]


def smaller_workloads(torch, np, datagen, vrl, dev, reps=12):
    """The four relayouts at the mid-size (P=2, 4,096 tokens/rank, 32 heads)
    and P=4 (7,752 tokens/rank, 32 heads) workloads and at one rank's share
    of the representative sequence over 4 and 8 ranks (13,854 and 6,927
    tokens per rank, 56 heads), rank 0's share.  Each op rotates over k
    copies of its buffers with k x bytes per launch >= 1 GiB, so every launch
    reads inputs that the previous launches have evicted from the 256 MB
    Infinity Cache; per-call HIP events and the queue's mean per call."""
    out = {}
    for w in [datagen.WORKLOADS[2], datagen.WORKLOADS[5]] + shard_workloads(datagen):
        P, C, S_l, H, D, G, S = w.P, w.C, w.s_local, w.H, w.D, w.G, w.S
        nb = op_bytes(w)
        bf = dict(dtype=torch.bfloat16, device=dev)
        host = datagen.fused_source(w, 0)
        fused0 = torch.from_numpy(host.view(np.int16)).to(dev).view(torch.bfloat16)
        k_big = _sets_for(nb["qkv_pack"], 64)
        k_small = _sets_for(nb["head_merge"], 64)
        sets = []
        for i in range(max(k_big, k_small)):
            fused = fused0.clone()
            packed = torch.empty(3 * S_l * H * D, **bf)
            vrl.qkv_pack(*[fused[:, j * H * D:(j + 1) * H * D].unflatten(1, (H, D)) for j in range(3)],
                         packed, P, C)
            sets.append({"qkv": [fused[:, j * H * D:(j + 1) * H * D].unflatten(1, (H, D)) for j in range(3)],
                         "packed": packed, "planes": [torch.empty(S, G, D, **bf) for _ in range(3)],
                         "send": torch.empty(S_l * H * D, **bf), "merged": torch.empty(S_l, H, D, **bf)})
        for st in sets:      # stand-ins for the received buffers, and a filled O
            vrl.qkv_unpack(st["packed"], *st["planes"], P, C)
        ops = {
            "qkv_pack": (k_big, lambda st: vrl.qkv_pack(*st["qkv"], st["packed"], P, C)),
            "qkv_unpack": (k_big, lambda st: vrl.qkv_unpack(st["packed"], *st["planes"], P, C)),
            "attn_split": (k_small, lambda st: vrl.attn_split(st["planes"][0], st["send"], P, C)),
            "head_merge": (k_small, lambda st: vrl.head_merge(st["send"], st["merged"], P, C)),
        }
        res = {"P": P, "C": C, "s_local": S_l, "H": H, "D": D}
        for name, (k, fn) in ops.items():
            for i in range(k):
                fn(sets[i])
            ts, mean = _queued(torch, fn, sets[:k], reps * k)
            res[name] = _stats(ts, mean, nb[name])
            res[name]["buffer_sets"] = k
        # the rotation must not have changed what the ops compute; the merge of
        # the split of the unpack of a rank's own packed buffer returns its Q
        ref = sets[0]
        for st in sets[1:]:
            if not (torch.equal(st["packed"].view(torch.int16), ref["packed"].view(torch.int16))
                    and torch.equal(st["merged"].view(torch.int16), ref["merged"].view(torch.int16))):
                raise SystemExit(f"{w.name}: buffer sets disagree")
        if not torch.equal(ref["merged"].view(torch.int16), ref["qkv"][0].view(torch.int16)):
            raise SystemExit(f"{w.name}: round trip is not bit-exact")
        out[w.name] = res
        del sets
    return out


def _sig(x, digits=4):
    """x rounded to `digits` significant digits (a small rate stays nonzero)."""
    return float(f"{x:.{digits}g}")


def cpu_baseline(w, hosts, nbytes, reps=21, single_reps=3):
    """The oracle's four chains for every rank (one step of the workload) on
    the host cores: one untimed pass, then `reps` timed passes; the median
    pass gives the rate."""
    import numpy as np

    import oracle

    d = oracle.dims(w.P, w.C, w.s_local, w.H, w.D)
    bufs = []
    for host in hosts:
        qkv = [host[:, i * w.H * w.D:(i + 1) * w.H * w.D].reshape(w.s_local, w.H, w.D)
               for i in range(3)]
        bufs.append((qkv, np.full(oracle.exchange_elems(d, 0), 0, dtype=np.uint16),
                     [np.full((w.S, w.G, w.D), 0, dtype=np.uint16) for _ in range(3)],
                     np.full(oracle.exchange_elems(d, 1), 0, dtype=np.uint16),
                     np.full((w.s_local, w.H, w.D), 0, dtype=np.uint16)))

    peaks = {}

    def one_pass():
        t = {"qkv_pack": 0.0, "qkv_unpack": 0.0, "attn_split": 0.0, "head_merge": 0.0}
        for qkv, packed, planes, send, merged in bufs:
            t0 = time.perf_counter()
            peaks["qkv_pack"] = oracle.qkv_pack(d, *qkv, packed)
            t1 = time.perf_counter()
            peaks["qkv_unpack"] = oracle.qkv_unpack(d, packed, *planes)
            t2 = time.perf_counter()
            peaks["attn_split"] = oracle.attn_split(d, planes[0], send)
            t3 = time.perf_counter()
            peaks["head_merge"] = oracle.head_merge(d, send, merged)
            t4 = time.perf_counter()
            t["qkv_pack"] += t1 - t0
            t["qkv_unpack"] += t2 - t1
            t["attn_split"] += t3 - t2
            t["head_merge"] += t4 - t3
        return t

    say("[bench] cpu baseline: untimed pass")
    one_pass()
    say(f"[bench] cpu baseline: {reps} timed passes")
    passes = sorted((one_pass() for _ in range(reps)), key=lambda t: sum(t.values()))
    med = passes[reps // 2]
    total = sum(med.values())
    cores = oracle.threads()
    result = {"value": _sig(len(hosts) * sum(nbytes.values()) / total / 1e9), "unit": "GB/s",
              "cores": cores, "kind": "oracle",
              "sample": f"one step of the workload (the pack, unpack, split and merge chains for each "
                        f"of the {len(hosts)} ranks, each rank's packed buffer standing in for its "
                        f"exchanged one); median of {reps} timed passes after one untimed pass",
              "ms": {k: round(1e3 * v, 1) for k, v in med.items()},
              "materialised_peak_bytes": dict(peaks)}
    # the same chains on one thread, one rank
    say(f"[bench] cpu baseline: one thread, one rank, {single_reps} passes")
    del bufs[1:]
    oracle.set_threads(1)
    try:
        singles = sorted((one_pass() for _ in range(single_reps)), key=lambda t: sum(t.values()))
    finally:
        oracle.set_threads(cores)
    t1 = singles[single_reps // 2]
    result["single_thread"] = {"value": _sig(sum(nbytes.values()) / sum(t1.values()) / 1e9), "unit": "GB/s",
                               "sample": f"rank 0's four chains, median of {single_reps} passes",
                               "ms": {k: round(1e3 * v, 1) for k, v in t1.items()}}
    return result


def read_traffic():
    """HBM bytes per QKV pack launch from the committed counter summary, or
    None when the kernel sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and not line.startswith("#"):
                fields[parts[0]] = parts[1]
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return int(fields["hbm_bytes_per_launch"])


# ---- counter runs --------------------------------------------------------------

# Kernels of the counter runs, in launch order: (label, op, kind).  Each is a
# distinct kernel instantiation, so per-kernel rows of a counter CSV map back
# to these labels.
PMC_KERNELS = [
    ("qkv_pack", "qkv_pack", "direct"),
    ("qkv_unpack", "qkv_unpack", "direct"),
    ("attn_split", "attn_split", "direct"),
    ("head_merge", "head_merge", "direct"),
    ("qkv_unpack head-major", "qkv_unpack", "head-run"),
    ("head_merge head-major", "head_merge", "head-run"),
    ("attn_split head-major", "attn_split", "direct strided-heads"),
]


def kernel_label(name):
    """(op, kind) of a relayout kernel's mangled-and-demangled name, or None."""
    if "(vrl::Op)" not in name:
        return None
    op = {"0": "qkv_pack", "1": "qkv_unpack", "2": "attn_split",
          "3": "head_merge"}[name.split("(vrl::Op)")[1][0]]
    if "headrun_kernel" in name:
        return op, "head-run"
    if "staged_kernel" in name:
        return op, "staged"
    if name.rstrip().endswith("false>(vrl::KernelArgs)"):
        return op, "direct strided-heads"
    return op, "direct"


def run_windows(args):
    """Only the one-chunk windows section, for a kernel trace of its own."""
    import numpy as np
    import torch

    import datagen
    import head_relayout_amd as vrl

    dev = torch.device("cuda:0")
    w = datagen.WORKLOADS[args.workload]
    say(f"[windows] workload {w.cid} ({w.name}): inputs for {w.P} ranks")
    ranks = [Rank(w, r, dev, torch, np, datagen, vrl) for r in range(w.P)]
    for rk in ranks:
        vrl.qkv_pack(*rk.qkv, rk.packed, w.P, w.C)
    exchange([rk.packed for rk in ranks], [rk.recv for rk in ranks], w.P)
    for rk in ranks:
        vrl.qkv_unpack(rk.recv, *rk.planes, w.P, w.C)
        vrl.attn_split(rk.planes[0], rk.send, w.P, w.C)
    exchange([rk.send for rk in ranks], [rk.back for rk in ranks], w.P)
    torch.cuda.synchronize()
    print(json.dumps({"workload": w.name, "windows": chunk_windows(torch, vrl, w, ranks)}), flush=True)


def run_pmc(args):
    """Every relayout kernel the representative shape uses (the four
    token-major ones, the head-run scatters into head-major views and the split
    from a head-major view) on rank 0's buffers, and a plain copy kernel,
    `reps` launches each."""
    import numpy as np
    import torch

    import datagen
    import head_relayout_amd as vrl

    dev = torch.device("cuda:0")
    w = datagen.WORKLOADS[args.workload]
    P, C = w.P, w.C
    rk = Rank(w, 0, dev, torch, np, datagen, vrl)
    bf = dict(dtype=torch.bfloat16, device=dev)
    vrl.qkv_pack(*rk.qkv, rk.packed, P, C)
    rk.recv.copy_(rk.packed)
    rk.back.copy_(rk.packed[:rk.back.numel()])
    hm = [torch.empty(w.G, w.S, w.D, **bf).transpose(0, 1) for _ in range(3)]
    merged_hm = torch.empty(w.H, w.s_local, w.D, **bf).transpose(0, 1)
    launches = {
        "qkv_pack": lambda: vrl.qkv_pack(*rk.qkv, rk.packed, P, C),
        "qkv_unpack": lambda: vrl.qkv_unpack(rk.recv, *rk.planes, P, C),
        "attn_split": lambda: vrl.attn_split(rk.planes[0], rk.send, P, C),
        "head_merge": lambda: vrl.head_merge(rk.back, rk.merged, P, C),
        "qkv_unpack head-major": lambda: vrl.qkv_unpack(rk.recv, *hm, P, C),
        "head_merge head-major": lambda: vrl.head_merge(rk.back, merged_hm, P, C),
        "attn_split head-major": lambda: vrl.attn_split(hm[0], rk.send, P, C),
    }
    n = rk.packed.numel()
    a = torch.zeros(n, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    for label, _, _ in PMC_KERNELS:
        for _ in range(args.reps):
            launches[label]()
    for _ in range(args.reps):
        torch.bitwise_not(a, out=b)     # reads n*2 bytes, writes n*2 bytes
    torch.cuda.synchronize()
    print(f"pmc: {args.reps} launches each of {len(PMC_KERNELS)} relayout kernels and of a "
          f"bitwise_not copy kernel ({2 * n} B read + written)", flush=True)


def run_pmc_sq(args):
    """The head-run unpack into head-major Q/K/V, the direct unpack into
    token-major ones and the pack, then the LDS-transpose kernels at head_dim
    16 and 32 (unpack into head-major Q/K/V, merge into a head-major output,
    split from a head-major O; 56 heads, the token count per rank scaled so
    every op moves the representative shape's bytes), `reps` launches each,
    for SQ counter runs."""
    import numpy as np
    import torch

    import datagen
    import head_relayout_amd as vrl

    dev = torch.device("cuda:0")
    w = datagen.WORKLOADS[args.workload]
    rk = Rank(w, 0, dev, torch, np, datagen, vrl)
    vrl.qkv_pack(*rk.qkv, rk.packed, w.P, w.C)
    rk.recv.copy_(rk.packed)
    hm = [torch.empty(w.G, w.S, w.D, dtype=torch.bfloat16, device=dev) for _ in range(3)]
    for _ in range(args.reps):
        vrl.qkv_unpack(rk.recv, *[t.transpose(0, 1) for t in hm], w.P, w.C)
    for _ in range(args.reps):
        vrl.qkv_unpack(rk.recv, *rk.planes, w.P, w.C)
    for _ in range(args.reps):
        vrl.qkv_pack(*rk.qkv, rk.packed, w.P, w.C)
    torch.cuda.synchronize()
    del rk, hm
    for D in (16, 32):
        n = datagen.Workload(0, f"{D}-element heads", P=w.P, C=w.C, s_local=w.s_local * w.D // D, H=w.H, D=D,
                             total_tokens=w.P * w.s_local * w.D // D, seed=w.seed)
        bf = dict(dtype=torch.bfloat16, device=dev)
        recv = torch.empty(3 * n.s_local * n.H * D, **bf)
        recv.view(torch.int16).random_(-30000, 30000)
        hm = [torch.empty(n.G, n.S, D, **bf) for _ in range(3)]
        out = torch.empty(n.H, n.s_local, D, **bf)
        send = torch.empty(n.s_local * n.H * D, **bf)
        for _ in range(args.reps):
            vrl.qkv_unpack(recv, *[t.transpose(0, 1) for t in hm], n.P, n.C)
        for _ in range(args.reps):
            vrl.head_merge(recv[:send.numel()], out.transpose(0, 1), n.P, n.C)
        for _ in range(args.reps):
            vrl.attn_split(hm[0].transpose(0, 1), send, n.P, n.C)
        torch.cuda.synchronize()
        del recv, hm, out, send
    print(f"pmc-sq: {args.reps} x head-run unpack (head-major), direct unpack, pack, and at head_dim 16 "
          f"and 32 the LDS-transpose unpack, merge and split (head-major)", flush=True)


def sq_summary(d):
    """Mean per-dispatch value of every counter in a --pmc tree, per kernel
    and grid (labelled with the workload when the grid is one this benchmark
    launches whole-tensor)."""
    whole = whole_tensor_grids()
    rows = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                lab = kernel_label(r["Kernel_Name"])
                if lab is None:
                    continue
                grid = int(r.get("Grid_Size") or r.get("Grid_Size_X") or 0)
                suffix = whole.get((lab[0], lab[1], grid), ("",))[0]
                rows.setdefault((lab[1] + " " + lab[0] + suffix, r["Counter_Name"]), []).append(
                    float(r["Counter_Value"]))
    kernels = sorted({k for k, _ in rows})
    counters = sorted({c for _, c in rows})
    print(f"{'kernel':<40}" + "".join(f"{c:>24}" for c in counters))
    for k in kernels:
        vals = [rows.get((k, c)) for c in counters]
        print(f"{k:<40}" + "".join(f"{(sum(v) / len(v) if v else float('nan')):24.0f}" for v in vals))


def pmc_summary(fetch_dir, write_dir):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of every relayout kernel of
    a --mode pmc run and of the copy kernel; the copy kernel's known size
    calibrates the counters.  The first two lines (source hash, pack bytes
    per launch) are what the benchmark's roofline reads."""
    def load(d, counter):
        rows = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") != counter:
                        continue
                    rows.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return rows

    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")

    def mean_of(rows, match):
        ks = [k for k in rows if match(k)]
        if len(ks) != 1:
            raise SystemExit(f"expected one kernel, found {ks} in {sorted(rows)}")
        vals = rows[ks[0]]
        return ks[0], sum(vals) / len(vals), len(vals)

    import datagen
    w = datagen.WORKLOADS[3]
    nb = op_bytes(w)
    copy_bytes = 3 * w.s_local * w.H * w.D * 2
    kc, cf, ncf = mean_of(fetch, lambda k: "bitwise_not" in k)
    _, cw, ncw = mean_of(write, lambda k: "bitwise_not" in k)
    f_scale = copy_bytes / (cf * 1024)
    w_scale = copy_bytes / (cw * 1024)
    table, pack_total = [], None
    for label, op, kind in PMC_KERNELS:
        def match(k, op=op, kind=kind):
            return kernel_label(k) == (op, kind)
        kname, f, nf = mean_of(fetch, match)
        _, wr, nw = mean_of(write, match)
        fb, wb = f * 1024 * f_scale, wr * 1024 * w_scale
        half = nb[op] // 2
        if label == "qkv_pack":
            pack_total = int(round(fb + wb))
        table.append(f"# {label:<24} {half:>14} {fb:>16.0f} {wb:>16.0f} {fb / half:>8.4f} {wb / half:>8.4f}"
                     f"   {nf}/{nw}")
    lines = [
        f"kernel_source_sha256 {kernel_source_hash()}",
        f"hbm_bytes_per_launch {pack_total}",
        f"# copy kernel: {kc}",
        f"#   FETCH_SIZE {cf:.1f} KiB/dispatch over {ncf}, WRITE_SIZE {cw:.1f} KiB/dispatch over {ncw}",
        f"#   known size {copy_bytes} B read and {copy_bytes} B written per dispatch",
        f"#   calibration: fetch x{f_scale:.4f}, write x{w_scale:.4f}",
        "# per launch, calibrated; algorithmic = bytes read = bytes written",
        f"# {'kernel':<24} {'algorithmic B':>14} {'fetched B':>16} {'written B':>16} {'fetch/x':>8} "
        f"{'write/x':>8}   dispatches",
    ] + table
    print("\n".join(lines))


# The launch planner's workgroup shapes (head_relayout_amd/csrc/vrl_internal.h),
# for labelling trace rows by grid size: lanes per workgroup and vectors per
# tile of the direct and head-run kernels, lanes of the LDS transpose.
DIRECT_THREADS, DIRECT_TILE = 64, 64
HEADRUN_THREADS, HEADRUN_TILE = 128, 256
STAGED_THREADS = 256


def whole_tensor_grids():
    """{(op, kind, grid in threads): (workload suffix, algorithmic bytes)} for
    the whole-tensor launches of the workloads this benchmark runs.  It
    follows the launch planner's tiling at 16-byte vectors: one-wave direct
    workgroups of 64 vectors, head-run workgroups of as many tokens of one
    head as fill 256 vectors."""
    import datagen

    out = {}
    shards = shard_workloads(datagen)
    for w, suffix in ((datagen.WORKLOADS[3], ""), (datagen.WORKLOADS[2], " (mid-size)"),
                      (datagen.WORKLOADS[5], " (P=4)"), (shards[0], " (P=4 shard)"), (shards[1], " (P=8 shard)")):
        nb = op_bytes(w)
        t_max = -(-w.s_local // w.C)
        head_vecs = w.D // 8
        row_vecs = w.G * head_vecs
        tt = min(HEADRUN_TILE // head_vecs, t_max)
        for op, nbytes in nb.items():
            blocks = w.P * w.C * (3 if op in ("qkv_pack", "qkv_unpack") else 1)
            direct = DIRECT_THREADS * blocks * -(-t_max * row_vecs // DIRECT_TILE)
            out[(op, "direct", direct)] = (suffix, nbytes)
            out[(op, "direct strided-heads", direct)] = (suffix, nbytes)
            out[(op, "head-run", HEADRUN_THREADS * blocks * w.G * -(-t_max // tt))] = (suffix, nbytes)
    # the representative shape with head chunks (rows of G / C heads, all S_l tokens)
    w = datagen.WORKLOADS[3]
    nb = op_bytes(w)
    hc_rows = -(-w.s_local * (w.G // w.C) * (w.D // 8) // DIRECT_TILE)
    for op, nbytes in nb.items():
        blocks = w.P * w.C * (3 if op in ("qkv_pack", "qkv_unpack") else 1)
        out.setdefault((op, "direct", DIRECT_THREADS * blocks * hc_rows), (" (head chunks)", nbytes))
    # the copy ceiling: a pack with P = 1, C = 1 of the representative shape
    w = datagen.WORKLOADS[3]
    out[("qkv_pack", "direct", DIRECT_THREADS * 3 * -(-w.s_local * w.H * w.D // 8 // DIRECT_TILE))] = (
        " (copy ceiling: P=1, C=1)", op_bytes(w)["qkv_pack"])
    # the narrow-head workloads (LDS transpose: a scatter's tiles of Gt heads
    # filling a 128-byte line x as many tokens as fit 8 KiB, a gather's of
    # the whole group x as many as fit 16 KiB, rounded to whole lines)
    base = datagen.WORKLOADS[3]
    for D in (16, 32):
        s_local = base.s_local * base.D // D
        t_max = -(-s_local // base.C)
        G, hv = base.G, D // 8
        quantum = max(1, 128 // (D * 2))
        for op in ("qkv_unpack", "attn_split", "head_merge"):
            # a gather's tiles hold the whole group, a scatter's a line's worth of heads
            gt = G if op == "attn_split" else next(g for g in range(1, G + 1) if G % g == 0 and g * D * 2 >= 128)
            tt = (16384 if op == "attn_split" else 8192) // (gt * hv * 16)
            tt = min(tt - tt % quantum, t_max)
            blocks = base.P * base.C * (3 if op == "qkv_unpack" else 1)
            nbytes = op_bytes(base)[op]
            key = (op, "staged", STAGED_THREADS * blocks * (G // gt) * -(-t_max // tt))
            label = f" (head_dim {D})" if key not in out else out[key][0][:-1] + f", {D})"
            out[key] = (label, nbytes)
    return out


def windows_summary(d):
    """Dispatch durations of the one-chunk window launches in a rocprofv3
    --kernel-trace run of `bench.py --mode windows` (representative shape):
    per op, all C windows together (same grid), with the rate on a window's
    mean algorithmic bytes (the op's bytes / C)."""
    import datagen

    paths = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    w = datagen.WORKLOADS[3]
    nb = op_bytes(w)
    t_max = -(-w.s_local // w.C)
    tiles = -(-t_max * (w.G * w.D // 8) // DIRECT_TILE)
    grid_of = {op: DIRECT_THREADS * w.P * (3 if op in ("qkv_pack", "qkv_unpack") else 1) * tiles for op in nb}
    times = {}
    with open(paths[0]) as f:
        for r in csv.DictReader(f):
            lab = kernel_label(r["Kernel_Name"])
            grid = int(r["Grid_Size_X"])
            if lab is None or lab[1] != "direct" or grid_of[lab[0]] != grid:
                continue
            times.setdefault(lab[0], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"# kernel sources: sha256 prefix {kernel_source_hash()}")
    print(f"# one-chunk windows [c, c+1), c = 0..{w.C - 1}, representative shape; bytes = the op's / {w.C}")
    print(f"{'op':<12} {'grid':>9} {'calls':>5} {'median_us':>10} {'p10_us':>8} {'p90_us':>8} {'avg_us':>8}"
          f" {'bytes':>11} {'GB/s(med)':>10} {'%8TB/s':>7}")
    for op in nb:
        ts = sorted(times.get(op, []))
        if not ts:
            continue
        n = len(ts)
        med = ts[n // 2]
        nbytes = nb[op] // w.C
        gbs = nbytes / (med * 1e-6) / 1e9
        print(f"{op:<12} {grid_of[op]:>9} {n:>5} {med:10.1f} {ts[n // 10]:8.1f} {ts[(9 * n) // 10]:8.1f}"
              f" {sum(ts) / n:8.1f} {nbytes:>11} {gbs:10.0f} {100 * gbs / PEAK_HBM_GBS:7.1f}")


def trace_summary(d):
    """Per-kernel table of a rocprofv3 --kernel-trace run of this benchmark,
    one row per (kernel, grid size)."""
    paths = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    groups = {}
    with open(paths[0]) as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], int(r["Grid_Size_X"]))
            groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    whole = whole_tensor_grids()
    print(f"# kernel sources: sha256 prefix {kernel_source_hash()}")
    print("# GB/s for whole-tensor launches (representative shape unless the label names")
    print("# another workload); \"(window)\" rows are chunk-window launches (the overlap")
    print("# schedule, the one-chunk split).")
    print(f"{'kernel':<40} {'grid':>9} {'calls':>5} {'avg_us':>9} {'min_us':>9} {'max_us':>9}"
          f" {'GB/s(avg)':>10} {'%8TB/s':>7}")
    for (name, grid), ns in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        avg = sum(ns) / len(ns)
        cols = f"{grid:>9} {len(ns):>5} {avg / 1e3:9.1f} {min(ns) / 1e3:9.1f} {max(ns) / 1e3:9.1f}"
        if kernel_label(name) is not None:
            op, kind = kernel_label(name)
            if (op, kind, grid) in whole:
                suffix, nbytes = whole[(op, kind, grid)]
                gbs = nbytes / (avg * 1e-9) / 1e9
                print(f"{kind + ' ' + op + suffix:<40} {cols} {gbs:10.0f} {100 * gbs / PEAK_HBM_GBS:7.1f}")
            else:
                print(f"{kind + ' ' + op + ' (window)':<40} {cols} {'-':>10} {'-':>7}")
        elif "copyBuffer" in name:
            print(f"{'__amd_rocclr_copyBuffer (exchanges)':<40} {cols}")


def main():
    args = parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.sq_summary:
        sq_summary(args.sq_summary)
        return
    if args.windows_summary:
        windows_summary(args.windows_summary)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the P ranks' "
              f"buffers and their exchange are modelled inside one GPU's HBM; a multi-GPU run "
              f"would exchange through RCCL and is not measured here.", file=sys.stderr)
        sys.exit(2)
    if args.mode == "pmc":
        run_pmc(args)
    elif args.mode == "windows":
        run_windows(args)
    elif args.mode == "pmc-sq":
        run_pmc_sq(args)
    else:
        run_bench(args)


if __name__ == "__main__":
    main()
