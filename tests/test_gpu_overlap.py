"""The four-chunk overlap schedule (per-chunk relayouts, exchanges on a
second stream, event-ordered ready waits) against the oracle: every buffer
the schedule writes -- packed, received, the three unpacked planes, the
split, the returned buffer and the merged output of every rank -- equals
the oracle's chains bit for bit, three runs in a row, with each of the three
stand-in exchanges (copy kernels, SDMA copies, link-paced copies).  The
serial schedule is checked against the same oracle buffers."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from datagen import WORKLOADS
from harness.ulysses import Layer, Rank, run_overlapped, run_serial
from tests.gpu_harness import SENTINEL, say, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "mid-size": WORKLOADS[2],
    "P=4 ragged": WORKLOADS[5],
    "representative": WORKLOADS[3],
}
ENGINES = ("kernel", "sdma", "link")
NAMES = ("packed", "recv", "plane q", "plane k", "plane v", "send", "back", "merged")


def _buffers(rk):
    return [rk.packed, rk.recv, *rk.planes, rk.send, rk.back, rk.merged]


def _oracle_layer(w, hosts, plane):
    """Every buffer of the layer computed by the oracle's chains, per rank in
    _buffers order: pack, exchange, unpack, split of one plane (attention is
    the identity here), exchange, merge."""
    P, C, S_l, H, D, G, S = w.P, w.C, w.s_local, w.H, w.D, w.G, w.S
    od = oracle.dims(P, C, S_l, H, D)
    packed = []
    for host in hosts:
        qkv = [host[:, i * H * D:(i + 1) * H * D].reshape(S_l, H, D) for i in range(3)]
        out = np.zeros(oracle.exchange_elems(od, 0), np.uint16)
        oracle.qkv_pack(od, *qkv, out)
        packed.append(out)
    recv = [np.zeros_like(x) for x in packed]
    oracle.exchange(od, 0, packed, recv)
    planes = []
    for r in range(P):
        ps = [np.zeros((S, G, D), np.uint16) for _ in range(3)]
        oracle.qkv_unpack(od, recv[r], *ps)
        planes.append(ps)
    send = []
    for r in range(P):
        out = np.zeros(oracle.exchange_elems(od, 1), np.uint16)
        oracle.attn_split(od, planes[r][plane], out)
        send.append(out)
    back = [np.zeros_like(x) for x in send]
    oracle.exchange(od, 1, send, back)
    merged = []
    for r in range(P):
        out = np.zeros((S_l, H, D), np.uint16)
        oracle.head_merge(od, back[r], out)
        merged.append(out)
    return [[packed[r], recv[r], *planes[r], send[r], back[r], merged[r]] for r in range(P)]


def _check(ranks, want, what):
    for r, rk in enumerate(ranks):
        for name, g, x in zip(NAMES, _buffers(rk), want[r]):
            assert torch.equal(g.reshape(-1).view(torch.int16), x.reshape(-1).view(torch.int16)), \
                f"{what}: rank {r}, {name} differs from the oracle"


@pytest.mark.parametrize("name", list(CASES))
def test_overlap_matches_oracle(gpu, name):
    w = CASES[name]
    plane = 1
    say(f"[overlap {name}] inputs and oracle buffers")
    hosts = [datagen.fused_source(w, r) for r in range(w.P)]
    want = [[to_dev(x, gpu) for x in per_rank] for per_rank in _oracle_layer(w, hosts, plane)]
    for r in range(w.P):   # the round trip returns the passed-through plane
        assert torch.equal(want[r][7].view(torch.int16),
                           to_dev(hosts[r], gpu)[:, plane * w.H * w.D:(plane + 1) * w.H * w.D]
                           .reshape(w.s_local, w.H, w.D).view(torch.int16))
    ranks = [Rank(to_dev(h, gpu), w.P, w.C, w.H, w.D) for h in hosts]
    comm = torch.cuda.Stream()
    for engine in ENGINES:
        layer = Layer(w.P, w.C, w.s_local, w.H, w.D, engine)
        say(f"[overlap {name}, {engine} exchange] serial")
        for rk in ranks:
            for b in _buffers(rk):
                b.view(torch.int16).fill_(SENTINEL)
        run_serial(layer, ranks, plane)
        torch.cuda.synchronize()
        _check(ranks, want, f"{name} ({engine}), serial schedule")
        for it in range(3):
            say(f"[overlap {name}, {engine} exchange] overlapped, run {it}")
            for rk in ranks:
                for b in _buffers(rk):
                    b.view(torch.int16).fill_(SENTINEL)
            torch.cuda.synchronize()
            run_overlapped(layer, ranks, comm, plane)
            torch.cuda.synchronize()
            _check(ranks, want, f"{name} ({engine}), overlapped run {it}")
    say(f"[overlap {name}] ok")
    del ranks, want
    torch.cuda.empty_cache()
