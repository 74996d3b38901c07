"""Edge cases of the HIP path against the CPU oracle, through the C ABI.

Ragged chunks, as many chunks as tokens, P = 1, 3, 4 and 8, one head per
group, small head_dims, padded source rows whose stride forces 2-, 4- and
8-byte vectors, a source base that is only 2-byte aligned, head-major and
padded output views, single-chunk windows, two concurrent streams, the
representative P=4 attention output read head-major, head_dims on both sides
of the 128-byte head-row threshold and beyond one tile, wide head groups,
4-D BTHD / BHTD tensors with B = 1 through the binding, and four host
threads calling at once.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import datagen
import head_relayout_amd as vrl
import oracle
from datagen import WORKLOADS
from tests.gpu_harness import (SENTINEL, assert_bits_equal, assert_guard_intact, guarded,
                               sentinel_view, to_dev)
from tests.pipeline import dev_qkv, host_qkv, run_pipeline

pytestmark = pytest.mark.gpu


def ids_fused(P, S_l, H, D, pad=0):
    """Per-rank fused sources holding distinct ids (never the sentinel)."""
    hd3 = 3 * H * D
    n = P * S_l * hd3
    assert n < 0xFFFF
    ids = np.arange(n, dtype=np.int64)
    ids[ids == SENTINEL] = 0xFFFF
    ids = ids.astype(np.uint16).reshape(P, S_l, hd3)
    out = []
    for r in range(P):
        f = np.full((S_l, hd3 + pad), SENTINEL, dtype=np.uint16)
        f[:, :hd3] = ids[r]
        out.append(f)
    return out


# (P, C, S_l, H, D, source row pad)
SHAPES = [
    (2, 1, 64, 4, 16, 0),
    (2, 4, 10, 4, 8, 0),
    (3, 2, 7, 6, 8, 0),
    (2, 5, 5, 4, 8, 0),
    (8, 3, 9, 8, 4, 0),
    (1, 2, 6, 3, 8, 0),
    (4, 4, 12, 8, 2, 3),
    (2, 3, 11, 4, 8, 1),      # odd row stride: 2-byte vectors
    (2, 3, 11, 4, 8, 2),      # 4-byte vectors
    (2, 3, 11, 4, 8, 4),      # 8-byte vectors
    (2, 3, 11, 4, 128, 8),    # 16-byte vectors, padded rows
    (2, 2, 9, 2, 200, 0),     # head_dim not a power of two, one head per group
    (2, 7, 40, 6, 24, 0),     # 3 heads per group of 24
    (2, 2, 6, 4, 1, 0),       # head_dim 1: one element per head row
    (3, 2, 7, 6, 3, 1),       # odd head_dim, padded rows
    (2, 3, 8, 4, 5, 0),       # odd head_dim, 2-byte vectors throughout
    (2, 2, 4, 4, 256, 0),     # head_dim 256
    (2, 3, 20, 4, 63, 0),     # 126-byte head rows: LDS transpose when head-major
    (2, 3, 20, 4, 64, 0),     # 128-byte head rows: head runs when head-major
]
IDS = [f"P{s[0]}C{s[1]}S{s[2]}H{s[3]}D{s[4]}pad{s[5]}" for s in SHAPES]


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
@pytest.mark.parametrize("layout", ["dense", "padded", "head_major"])
def test_small_shapes(gpu, shape, layout):
    P, C, S_l, H, D, pad = shape
    lay = {"dense": {}, "padded": {"row_pad": 5}, "head_major": {"head_major": True}}[layout]
    run_pipeline(gpu, P, C, S_l, H, D, ids_fused(P, S_l, H, D, pad), f"{IDS[SHAPES.index(shape)]}-{layout}",
                 unpack_layout=lay, merge_layout=lay)


@pytest.mark.parametrize("offset", [1, 2, 4])
def test_source_base_alignment(gpu, offset):
    """A fused source starting 2, 4 or 8 bytes past a 16-byte boundary."""
    P, C, S_l, H, D = 2, 4, 33, 4, 64
    run_pipeline(gpu, P, C, S_l, H, D, ids_fused(P, S_l, H, D), f"offset{offset}",
                 base_offset=offset, planes=(1,))


def _window_case(gpu, P, C, S_l, H, D, tag):
    G, S = H // P, P * S_l
    od = oracle.dims(P, C, S_l, H, D)
    rng = np.random.default_rng(7)
    fused = rng.integers(0, 0x7F00, size=(S_l, 3 * H * D), dtype=np.uint16)
    dq = dev_qkv(to_dev(fused, gpu), H, D)
    n_qkv = vrl.exchange_elems(0, P, C, S_l, H, D)
    n_att = vrl.exchange_elems(1, P, C, S_l, H, D)
    acc, acc_whole = guarded(n_qkv, gpu)
    for c in range(C):
        one, _ = guarded(n_qkv, gpu)
        vrl.qkv_pack(*dq, one, P, C, c, c + 1)
        vrl.qkv_pack(*dq, acc, P, C, c, c + 1)
        ref = np.full(n_qkv, SENTINEL, dtype=np.uint16)
        oracle.qkv_pack(od, *host_qkv(fused, H, D), ref, c, c + 1)
        torch.cuda.synchronize()
        assert_bits_equal(one, ref, f"{tag} pack window {c}")
    full = np.zeros(n_qkv, dtype=np.uint16)
    oracle.qkv_pack(od, *host_qkv(fused, H, D), full)
    assert_bits_equal(acc, full, f"{tag} pack windows composed")
    assert_guard_intact(acc_whole, f"{tag} pack windows")

    recv = acc
    outs = [sentinel_view(S, G, D, gpu) for _ in range(3)]
    for c in range(C):
        vrl.qkv_unpack(recv, *[o[0] for o in outs], P, C, c, c + 1)
        ref = [np.full((S, G, D), SENTINEL, dtype=np.uint16) for _ in range(3)]
        for cc in range(c + 1):
            oracle.qkv_unpack(od, full, *ref, cc, cc + 1)
        torch.cuda.synchronize()
        for i in range(3):
            assert_bits_equal(outs[i][0], ref[i], f"{tag} unpack after window {c} plane {i}")

    o_ref = np.zeros((S, G, D), dtype=np.uint16)
    oracle.qkv_unpack(od, full, o_ref, np.zeros_like(o_ref), np.zeros_like(o_ref))
    send, _ = guarded(n_att, gpu)
    for c in range(C):
        vrl.attn_split(outs[0][0], send, P, C, c, c + 1)
        ref = np.full(n_att, SENTINEL, dtype=np.uint16)
        for cc in range(c + 1):
            oracle.attn_split(od, o_ref, ref, cc, cc + 1)
        torch.cuda.synchronize()
        assert_bits_equal(send, ref, f"{tag} split after window {c}")

    ref_send = np.zeros(n_att, dtype=np.uint16)
    oracle.attn_split(od, o_ref, ref_send)
    out, whole = sentinel_view(S_l, H, D, gpu, row_pad=3)
    for c in range(C):
        vrl.head_merge(send, out, P, C, c, c + 1)
        ref = np.full((S_l, H, D), SENTINEL, dtype=np.uint16)
        for cc in range(c + 1):
            oracle.head_merge(od, ref_send, ref, cc, cc + 1)
        torch.cuda.synchronize()
        assert_bits_equal(out, ref, f"{tag} merge after window {c}")
    assert_guard_intact(whole, f"{tag} merge windows")


def test_windows_ragged(gpu):
    _window_case(gpu, 3, 4, 10, 6, 8, "windows ragged")


def test_windows_mid_size(gpu):
    w = WORKLOADS[2]
    _window_case(gpu, w.P, w.C, w.s_local, w.H, w.D, "windows mid-size")


def test_two_streams(gpu):
    """Two ranks' packs and merges enqueued concurrently on two streams."""
    w = WORKLOADS[2]
    P, C, S_l, H, D = w.P, w.C, w.s_local, w.H, w.D
    od = oracle.dims(P, C, S_l, H, D)
    fused = [datagen.fused_source(w, r) for r in range(P)]
    dev = [to_dev(f, gpu) for f in fused]
    n = vrl.exchange_elems(0, P, C, S_l, H, D)
    outs = [torch.empty(n, dtype=torch.bfloat16, device=gpu) for _ in range(P)]
    merged = [torch.empty(S_l, H, D, dtype=torch.bfloat16, device=gpu) for _ in range(P)]
    recv_att = [to_dev(datagen.values(S_l * H * D, seed=9, stream=r), gpu) for r in range(P)]
    streams = [torch.cuda.Stream() for _ in range(P)]
    torch.cuda.synchronize()
    for _ in range(3):
        for r in range(P):
            vrl.qkv_pack(*dev_qkv(dev[r], H, D), outs[r], P, C, stream=streams[r])
            vrl.head_merge(recv_att[r], merged[r], P, C, stream=streams[r])
    torch.cuda.synchronize()
    for r in range(P):
        ref = np.zeros(n, dtype=np.uint16)
        oracle.qkv_pack(od, *host_qkv(fused[r], H, D), ref)
        assert_bits_equal(outs[r], ref, f"two streams pack rank {r}")
        m = np.zeros((S_l, H, D), dtype=np.uint16)
        oracle.head_merge(od, recv_att[r].view(torch.int16).cpu().numpy().view(np.uint16), m)
        assert_bits_equal(merged[r], m, f"two streams merge rank {r}")


@pytest.mark.parametrize("head_major", [False, True])
def test_split_config5_attention_output(gpu, head_major):
    """The P=4 workload's per-rank [31,008][8][128] attention output, read
    contiguous and head-major (BHTD storage)."""
    w = WORKLOADS[5]
    P, C, S_l, H, D, G, S = w.P, w.C, w.s_local, w.H, w.D, w.G, w.S
    od = oracle.dims(P, C, S_l, H, D)
    n_att = vrl.exchange_elems(1, P, C, S_l, H, D)
    for r in range(P):
        o = datagen.attention_output(w, r)              # [S][G][D]
        if head_major:
            dev_o = to_dev(np.ascontiguousarray(o.transpose(1, 0, 2)), gpu).transpose(0, 1)
        else:
            dev_o = to_dev(o, gpu)
        send, whole = guarded(n_att, gpu)
        vrl.attn_split(dev_o, send, P, C)
        ref = np.zeros(n_att, dtype=np.uint16)
        oracle.attn_split(od, o, ref)
        torch.cuda.synchronize()
        assert_bits_equal(send, ref, f"cfg5 split rank {r} head_major={head_major}")
        assert_guard_intact(whole, "cfg5 split")


@pytest.mark.parametrize("layout", ["dense", "head_major"])
def test_wide_head_groups(gpu, layout):
    """66 heads of 128 per group (16,896-byte wire rows), 200 tokens per rank:
    head-major scatters run as head runs over 66 heads, with ragged chunks
    and a partial last token tile.  Random payloads (the shape has more
    elements than unique 16-bit ids)."""
    P, C, S_l, H, D = 2, 3, 200, 132, 128
    rng = np.random.default_rng(66)
    fused = [rng.integers(0, 0x7F00, size=(S_l, 3 * H * D), dtype=np.uint16) for _ in range(P)]
    lay = {"dense": {}, "head_major": {"head_major": True}}[layout]
    run_pipeline(gpu, P, C, S_l, H, D, fused, f"wide-groups-{layout}", unpack_layout=lay, merge_layout=lay)


@pytest.mark.parametrize("layout", ["dense", "head_major"])
def test_head_rows_longer_than_a_tile(gpu, layout):
    """head_dim 16,392 (2,049 vectors of 16 bytes per head row, more than one
    workgroup tile): head-major views then fall back to wire order."""
    P, C, S_l, H, D = 2, 2, 3, 4, 16392
    rng = np.random.default_rng(16392)
    fused = [rng.integers(0, 0x7F00, size=(S_l, 3 * H * D), dtype=np.uint16) for _ in range(P)]
    lay = {"dense": {}, "head_major": {"head_major": True}}[layout]
    run_pipeline(gpu, P, C, S_l, H, D, fused, f"long-heads-{layout}", unpack_layout=lay, merge_layout=lay)


def test_bthd_tensors_with_batch_one(gpu):
    """The binding takes BTHD tensors [1][S][G][D] (B = 1) as well as
    [S][G][D]: unpack into, and split from, 4-D tensors, including a
    head-major BHTD one viewed as BTHD."""
    w = WORKLOADS[1]
    P, C, S_l, H, D, G, S = w.P, w.C, w.s_local, w.H, w.D, w.G, w.S
    od = oracle.dims(P, C, S_l, H, D)
    n = vrl.exchange_elems(vrl.VRL_EXCHANGE_QKV, P, C, S_l, H, D)
    recv = datagen.values(n, seed=21, stream=0)
    drecv = to_dev(recv, gpu)
    bthd = [torch.empty(1, S, G, D, dtype=torch.bfloat16, device=gpu) for _ in range(3)]
    bhtd = [torch.empty(1, G, S, D, dtype=torch.bfloat16, device=gpu) for _ in range(3)]
    vrl.qkv_unpack(drecv, *bthd, P, C)
    vrl.qkv_unpack(drecv, *[t.transpose(1, 2) for t in bhtd], P, C)
    want = [np.zeros((S, G, D), dtype=np.uint16) for _ in range(3)]
    oracle.qkv_unpack(od, recv, *want)
    torch.cuda.synchronize()
    for q in range(3):
        assert_bits_equal(bthd[q][0], want[q], f"BTHD unpack plane {q}")
        assert_bits_equal(bhtd[q][0].transpose(0, 1), want[q], f"BHTD unpack plane {q}")
    send = torch.empty(vrl.exchange_elems(vrl.VRL_EXCHANGE_ATTN, P, C, S_l, H, D), dtype=torch.bfloat16,
                       device=gpu)
    ref = np.zeros(send.numel(), dtype=np.uint16)
    oracle.attn_split(od, want[2], ref)
    for o in (bthd[2], bhtd[2].transpose(1, 2)):
        send.zero_()
        vrl.attn_split(o, send, P, C)
        torch.cuda.synchronize()
        assert_bits_equal(send, ref, "split from a 4-D tensor")


def test_concurrent_host_threads(gpu):
    """Four host threads, each with its own stream, pack and merge distinct
    inputs at the same time (ctypes drops the GIL inside the library): every
    result equals the oracle's."""
    import threading

    w = WORKLOADS[1]
    P, C, S_l, H, D = w.P, w.C, w.s_local, w.H, w.D
    od = oracle.dims(P, C, S_l, H, D)
    n_qkv = vrl.exchange_elems(vrl.VRL_EXCHANGE_QKV, P, C, S_l, H, D)
    n_att = vrl.exchange_elems(vrl.VRL_EXCHANGE_ATTN, P, C, S_l, H, D)
    hosts = [datagen.values(S_l * 3 * H * D, seed=40 + t, stream=0).reshape(S_l, 3 * H * D) for t in range(4)]
    backs = [datagen.values(n_att, seed=50 + t, stream=0) for t in range(4)]
    fused = [to_dev(h, gpu) for h in hosts]
    dback = [to_dev(b, gpu) for b in backs]
    packed = [torch.empty(n_qkv, dtype=torch.bfloat16, device=gpu) for _ in range(4)]
    merged = [torch.empty(S_l, H, D, dtype=torch.bfloat16, device=gpu) for _ in range(4)]
    streams = [torch.cuda.Stream() for _ in range(4)]
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            torch.cuda.set_device(gpu)
            for _ in range(50):
                vrl.qkv_pack(*dev_qkv(fused[t], H, D), packed[t], P, C, stream=streams[t])
                vrl.head_merge(dback[t], merged[t], P, C, stream=streams[t])
            streams[t].synchronize()
        except Exception as e:          # reported by the main thread
            errors.append(f"thread {t}: {e}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for t in range(4):
        ref = np.zeros(n_qkv, dtype=np.uint16)
        oracle.qkv_pack(od, *host_qkv(hosts[t], H, D), ref)
        assert_bits_equal(packed[t], ref, f"thread {t} pack")
        m = np.zeros((S_l, H, D), dtype=np.uint16)
        oracle.head_merge(od, backs[t], m)
        assert_bits_equal(merged[t], m, f"thread {t} merge")
