"""The reference materialisation arm (harness/reference_chains.py: the torch
chains the direct relayouts replace, run on the GPU) against the oracle, and
its allocation peaks against the allocation screen of Vflash's "Sol-Engine
alignment on SM86 and SM89" page ("What is enabled", the paragraph after the
operation table; fixture tests/golden/allocation_screen.txt)."""
import numpy as np
import pytest
import torch

import datagen
import head_relayout_amd as vrl
import oracle
from datagen import WORKLOADS
from harness import reference_chains as rc
from tests.gpu_harness import assert_bits_equal, say, to_dev
from tests.golden.load import load

pytestmark = pytest.mark.gpu


def _host_qkv(host, S_l, H, D):
    return [host[:, i * H * D:(i + 1) * H * D].reshape(S_l, H, D) for i in range(3)]


def _dev_qkv(dev_fused, H, D):
    return [dev_fused[:, i * H * D:(i + 1) * H * D].unflatten(1, (H, D)) for i in range(3)]


@pytest.mark.parametrize("wid", [1, 2])
def test_reference_chains_match_oracle(gpu, wid):
    """Every chain's output, element for element, at the tiny round-trip and
    mid-size workloads; the split also one chunk window at a time."""
    w = WORKLOADS[wid]
    P, C, S_l, H, D, G, S = w.P, w.C, w.s_local, w.H, w.D, w.G, w.S
    od = oracle.dims(P, C, S_l, H, D)
    hosts = [datagen.fused_source(w, r) for r in range(P)]
    tag = f"workload {wid}"
    say(f"[reference arm {tag}] pack")
    packed = []
    for r in range(P):
        want = np.zeros(oracle.exchange_elems(od, 0), np.uint16)
        oracle.qkv_pack(od, *_host_qkv(hosts[r], S_l, H, D), want)
        got = rc.ref_pack(torch, *_dev_qkv(to_dev(hosts[r], gpu), H, D), P, C)
        assert_bits_equal(got, want, f"{tag} reference pack rank {r}")
        packed.append(want)
    recv = [np.zeros_like(x) for x in packed]
    oracle.exchange(od, 0, packed, recv)
    say(f"[reference arm {tag}] unpack")
    planes = []
    for r in range(P):
        want = [np.zeros((S, G, D), np.uint16) for _ in range(3)]
        oracle.qkv_unpack(od, recv[r], *want)
        got = rc.ref_unpack(torch, to_dev(recv[r], gpu), P, C, S_l, G, D)
        for q in range(3):
            assert_bits_equal(got[q], want[q], f"{tag} reference unpack rank {r} plane {q}")
        planes.append(want)
    say(f"[reference arm {tag}] split, whole and per chunk window")
    sends = []
    for r in range(P):
        o = planes[r][0]
        want = np.zeros(oracle.exchange_elems(od, 1), np.uint16)
        oracle.attn_split(od, o, want)
        do = to_dev(o, gpu)
        assert_bits_equal(rc.ref_split(torch, do, P, C), want, f"{tag} reference split rank {r}")
        # a window's output is its (dest, chunk) blocks back to back, dest-major
        lens = [len(x) for x in torch.tensor_split(torch.arange(S_l), C)]
        off = [sum(lens[:c]) for c in range(C + 1)]
        for c in range(C):
            blocks = [want[(d * S_l + off[c]) * G * D:(d * S_l + off[c + 1]) * G * D] for d in range(P)]
            assert_bits_equal(rc.ref_split(torch, do, P, C, c, c + 1), np.concatenate(blocks),
                              f"{tag} reference split rank {r} chunk {c}")
        sends.append(want)
    back = [np.zeros_like(x) for x in sends]
    oracle.exchange(od, 1, sends, back)
    say(f"[reference arm {tag}] merge")
    for r in range(P):
        want = np.zeros((S_l, H, D), np.uint16)
        oracle.head_merge(od, back[r], want)
        got = rc.ref_merge(torch, to_dev(back[r], gpu), P, S_l, G, D)
        assert_bits_equal(got, want, f"{tag} reference merge rank {r}")
        assert_bits_equal(got, _host_qkv(hosts[r], S_l, H, D)[0], f"{tag} reference round trip rank {r}")
    say(f"[reference arm {tag}] ok")


def test_reference_peaks_match_allocation_screen(gpu):
    """At the representative shape the reference chains peak at exactly twice
    the direct relayouts' outputs -- 2,383,245,312 vs 1,191,622,656 B (pack),
    794,415,104 vs 397,207,552 B (merge) -- and a one-chunk split window
    holds 94.7 MiB, as the page's allocation screen prints.  The chains'
    pack and merge outputs are also compared with the oracle's."""
    g = load("allocation_screen.txt")
    w = WORKLOADS[3]
    P, C, S_l, H, D, G = w.P, w.C, w.s_local, w.H, w.D, w.G
    od = oracle.dims(P, C, S_l, H, D)
    say("[reference arm representative] inputs")
    host = datagen.fused_source(w, 0)
    qkv = _dev_qkv(to_dev(host, gpu), H, D)
    back_host = datagen.values(S_l * H * D, seed=w.seed, stream=200)
    back = to_dev(back_host, gpu)
    o = torch.empty(w.S, G, D, dtype=torch.bfloat16, device=gpu)
    o.view(torch.int16).random_(-30000, 30000)
    bf = dict(dtype=torch.bfloat16, device=gpu)

    def d_pack():
        out = torch.empty(3 * S_l * H * D, **bf)
        vrl.qkv_pack(*qkv, out, P, C)
        return out

    def d_merge():
        out = torch.empty(S_l, H, D, **bf)
        vrl.head_merge(back, out, P, C)
        return out

    say("[reference arm representative] peaks")
    assert rc.peak_bytes(torch, lambda: rc.ref_pack(torch, *qkv, P, C)) == g["pack_reference_peak_bytes"]
    assert rc.peak_bytes(torch, d_pack) == g["pack_direct_peak_bytes"]
    assert rc.peak_bytes(torch, lambda: rc.ref_merge(torch, back, P, S_l, G, D)) == g["merge_reference_peak_bytes"]
    assert rc.peak_bytes(torch, d_merge) == g["merge_direct_peak_bytes"]
    split_peak = rc.peak_bytes(torch, lambda: rc.ref_split(torch, o, P, C, 0, 1))
    assert round(split_peak / 2 ** 20, 1) == g["split_output_mib"]
    assert split_peak == P * len(torch.tensor_split(torch.arange(S_l), C)[0]) * G * D * 2

    say("[reference arm representative] outputs against the oracle")
    want = np.zeros(oracle.exchange_elems(od, 0), np.uint16)
    oracle.qkv_pack(od, *_host_qkv(host, S_l, H, D), want)
    assert_bits_equal(rc.ref_pack(torch, *qkv, P, C), want, "representative reference pack")
    assert_bits_equal(d_pack(), want, "representative direct pack")
    want = np.zeros((S_l, H, D), np.uint16)
    oracle.head_merge(od, back_host, want)
    assert_bits_equal(rc.ref_merge(torch, back, P, S_l, G, D), want, "representative reference merge")
    assert_bits_equal(d_merge(), want, "representative direct merge")
    say("[reference arm representative] ok")
