"""The whole relayout path on the GPU, stage by stage against the oracle.

For P ranks: pack -> exchange -> unpack -> split(O := an unpacked plane) ->
exchange -> merge, for each of the planes asked for.  Every stage's device
output is compared bit for bit with the oracle's output for the same input;
every device output lives in a sentinel-filled allocation whose guard bands
and padding are checked untouched; the merge must return the source plane.
"""
from __future__ import annotations

import numpy as np
import torch

import head_relayout_amd as vrl
import oracle
from tests.gpu_harness import (assert_bits_equal, assert_guard_intact, guarded, say,
                               sentinel_view, sim_exchange, to_dev)


def host_qkv(fused: np.ndarray, H: int, D: int):
    S_l = fused.shape[0]
    return [fused[:, i * H * D:(i + 1) * H * D].reshape(S_l, H, D) for i in range(3)]


def dev_qkv(fused: torch.Tensor, H: int, D: int):
    return [fused[:, i * H * D:(i + 1) * H * D].unflatten(1, (H, D)) for i in range(3)]


def run_pipeline(dev, P, C, S_l, H, D, fused, tag, planes=(0, 1, 2), unpack_layout=None,
                 merge_layout=None, base_offset=0, chunk_heads=False):
    """fused: per-rank host uint16 [S_l][3*H*D + pad] sources.
    unpack_layout / merge_layout: dict(row_pad=.., head_major=..) of the
    device output views.  base_offset: elements by which every device source
    is shifted inside its allocation (to exercise narrow alignments).
    chunk_heads: chunks split head groups instead of tokens."""
    hc = dict(chunk_heads=chunk_heads)
    unpack_layout = unpack_layout or {}
    merge_layout = merge_layout or {}
    G, S = H // P, P * S_l
    od = oracle.dims(P, C, S_l, H, D)
    n_qkv = vrl.exchange_elems(vrl.VRL_EXCHANGE_QKV, P, C, S_l, H, D, **hc)
    n_att = vrl.exchange_elems(vrl.VRL_EXCHANGE_ATTN, P, C, S_l, H, D, **hc)

    dfused = []
    for f in fused:
        flat = to_dev(np.concatenate([np.zeros(base_offset, np.uint16), f.reshape(-1)]), dev)
        dfused.append(flat[base_offset:].view(f.shape))

    say(f"[{tag}] pack")
    packed, ref_packed = [], []
    for r in range(P):
        inner, whole = guarded(n_qkv, dev)
        vrl.qkv_pack(*dev_qkv(dfused[r], H, D), inner, P, C, **hc)
        ref = np.zeros(n_qkv, dtype=np.uint16)
        oracle.qkv_pack(od, *host_qkv(fused[r], H, D), ref, **hc)
        torch.cuda.synchronize()
        assert_bits_equal(inner, ref, f"{tag} pack rank {r}")
        assert_guard_intact(whole, f"{tag} pack rank {r}")
        packed.append(inner)
        ref_packed.append(ref)

    recv = [torch.empty_like(p) for p in packed]
    sim_exchange(packed, recv, P)
    ref_recv = [np.zeros(n_qkv, dtype=np.uint16) for _ in range(P)]
    oracle.exchange(od, 0, ref_packed, ref_recv, **hc)
    del ref_packed, packed
    for r in range(P):
        assert_bits_equal(recv[r], ref_recv[r], f"{tag} simulated exchange rank {r}")

    say(f"[{tag}] unpack")
    unpacked = []
    for r in range(P):
        outs = [sentinel_view(S, G, D, dev, **unpack_layout) for _ in range(3)]
        vrl.qkv_unpack(recv[r], *[o[0] for o in outs], P, C, **hc)
        ref = [np.zeros((S, G, D), dtype=np.uint16) for _ in range(3)]
        oracle.qkv_unpack(od, ref_recv[r], *ref, **hc)
        torch.cuda.synchronize()
        for i in range(3):
            assert_bits_equal(outs[i][0], ref[i], f"{tag} unpack rank {r} plane {i}")
            # sentinel padding and guard bands untouched
            whole = outs[i][1]
            n_written = S * G * D
            sentinels = int((whole.view(torch.int16) == 0x7FC1).sum())
            assert sentinels == whole.numel() - n_written, f"{tag} unpack rank {r}: padding written"
            assert_guard_intact(whole, f"{tag} unpack rank {r} plane {i}")
        unpacked.append((outs, ref))
    del recv, ref_recv

    for qi in planes:
        say(f"[{tag}] split + merge, plane {qi}")
        sends, ref_sends = [], []
        for r in range(P):
            o_dev, o_ref = unpacked[r][0][qi][0], unpacked[r][1][qi]
            inner, whole = guarded(n_att, dev)
            vrl.attn_split(o_dev, inner, P, C, **hc)
            ref = np.zeros(n_att, dtype=np.uint16)
            oracle.attn_split(od, o_ref, ref, **hc)
            torch.cuda.synchronize()
            assert_bits_equal(inner, ref, f"{tag} split rank {r} plane {qi}")
            assert_guard_intact(whole, f"{tag} split rank {r} plane {qi}")
            sends.append(inner)
            ref_sends.append(ref)
        back = [torch.empty_like(s) for s in sends]
        sim_exchange(sends, back, P)
        ref_back = [np.zeros(n_att, dtype=np.uint16) for _ in range(P)]
        oracle.exchange(od, 1, ref_sends, ref_back, **hc)
        for r in range(P):
            out, whole = sentinel_view(S_l, H, D, dev, **merge_layout)
            vrl.head_merge(back[r], out, P, C, **hc)
            ref = np.zeros((S_l, H, D), dtype=np.uint16)
            oracle.head_merge(od, ref_back[r], ref, **hc)
            torch.cuda.synchronize()
            assert_bits_equal(out, ref, f"{tag} merge rank {r} plane {qi}")
            assert_bits_equal(out, host_qkv(fused[r], H, D)[qi], f"{tag} round trip rank {r} plane {qi}")
            n_written = S_l * H * D
            sentinels = int((whole.view(torch.int16) == 0x7FC1).sum())
            assert sentinels == whole.numel() - n_written, f"{tag} merge rank {r}: padding written"
            assert_guard_intact(whole, f"{tag} merge rank {r} plane {qi}")
    say(f"[{tag}] ok")
