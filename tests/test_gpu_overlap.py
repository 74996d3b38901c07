"""The four-chunk overlap schedule (per-chunk relayouts, exchanges on a
second stream, event-ordered ready waits) against the serial schedule:
every wire buffer and output identical bit for bit, three runs in a row,
and the round trip returning the input plane."""
import numpy as np
import pytest
import torch

import datagen
from datagen import WORKLOADS
from harness.ulysses import Layer, Rank, run_overlapped, run_serial
from tests.gpu_harness import SENTINEL, say, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "mid-size": WORKLOADS[2],
    "P=4 ragged": WORKLOADS[5],
    "representative": WORKLOADS[3],
}


def _buffers(rk):
    return [rk.packed, rk.recv, *rk.planes, rk.send, rk.back, rk.merged]


@pytest.mark.parametrize("engine", ["kernel", "sdma"])
@pytest.mark.parametrize("name", list(CASES))
def test_overlap_matches_serial(gpu, name, engine):
    """engine: the stand-in exchange as copy kernels or as SDMA copies."""
    w = CASES[name]
    say(f"[overlap {name}, {engine} exchange] inputs")
    layer = Layer(w.P, w.C, w.s_local, w.H, w.D, engine)
    ranks = [Rank(to_dev(datagen.fused_source(w, r), gpu), w.P, w.C, w.H, w.D) for r in range(w.P)]
    plane = 1
    run_serial(layer, ranks, plane)
    torch.cuda.synchronize()
    want = [[b.clone() for b in _buffers(rk)] for rk in ranks]
    for rk in ranks:
        assert torch.equal(rk.merged.view(torch.int16), rk.qkv[plane].view(torch.int16))
    comm = torch.cuda.Stream()
    for it in range(3):
        for rk in ranks:
            for b in _buffers(rk):
                b.view(torch.int16).fill_(SENTINEL)
        torch.cuda.synchronize()
        run_overlapped(layer, ranks, comm, plane)
        torch.cuda.synchronize()
        for r, rk in enumerate(ranks):
            for i, (g, x) in enumerate(zip(_buffers(rk), want[r])):
                assert torch.equal(g.view(torch.int16), x.view(torch.int16)), \
                    f"{name} ({engine}): run {it}, rank {r}, buffer {i} differs from the serial schedule"
    say(f"[overlap {name}, {engine} exchange] ok")
    del ranks, want
    torch.cuda.empty_cache()
