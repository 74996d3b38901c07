"""The relayouts captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
every replay, with eager work and synchronisation between replays and the
inputs changed in between, must equal the eager calls bit for bit."""
import numpy as np
import pytest
import torch

import datagen
import head_relayout_amd as vrl
from datagen import WORKLOADS
from harness.ulysses import Layer, Rank
from tests.gpu_harness import to_dev

pytestmark = pytest.mark.gpu


def _step(ranks, P, C, chunk_heads=False):
    hc = dict(chunk_heads=chunk_heads)
    for rk in ranks:
        vrl.qkv_pack(*rk.qkv, rk.packed, P, C, **hc)
        vrl.qkv_unpack(rk.recv, *rk.planes, P, C, **hc)
        vrl.attn_split(rk.planes[0], rk.send, P, C, **hc)
        vrl.head_merge(rk.back, rk.merged, P, C, **hc)


def _outs(ranks):
    return [t.clone() for rk in ranks for t in (rk.packed, *rk.planes, rk.send, rk.merged)]


@pytest.mark.parametrize("chunk_heads,layout", [(False, "token-major"), (True, "token-major"),
                                                 (False, "head-major"), (False, "head-major, D=16")])
def test_graph_replays_match_eager(gpu, chunk_heads, layout):
    """Token-major views run the direct kernel; head-major attention side and
    merge output the head-run kernel, or with 16-element heads the LDS
    transpose."""
    w = WORKLOADS[2]
    if layout == "head-major, D=16":
        w = datagen.Workload(0, "mid-size, 16-element heads", P=w.P, C=w.C, s_local=w.s_local, H=w.H, D=16,
                             total_tokens=w.total_tokens, seed=w.seed)
    P, C = w.P, w.C
    ranks = [Rank(to_dev(datagen.fused_source(w, r), gpu), P, C, w.H, w.D) for r in range(P)]
    if layout != "token-major":
        for rk in ranks:
            bf = dict(dtype=torch.bfloat16, device=gpu)
            rk.planes = [torch.empty(w.G, w.S, w.D, **bf).transpose(0, 1) for _ in range(3)]
            rk.merged = torch.empty(w.H, w.s_local, w.D, **bf).transpose(0, 1)
    rng = np.random.default_rng(5)

    def refill(seed):
        for r, rk in enumerate(ranks):
            rk.recv.copy_(to_dev(datagen.values(rk.recv.numel(), seed=seed, stream=r), gpu))
            rk.back.copy_(to_dev(datagen.values(rk.back.numel(), seed=seed, stream=10 + r), gpu))
            rk.fused.copy_(to_dev(datagen.fused_source(w, r), gpu) if seed == 0 else
                           to_dev(rng.integers(0, 0x7F00, size=tuple(rk.fused.shape), dtype=np.uint16), gpu))

    refill(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm-up on a side stream, as capture requires
        _step(ranks, P, C, chunk_heads)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(ranks, P, C, chunk_heads)
    torch.cuda.synchronize()
    for it in range(4):
        refill(it + 1)
        torch.cuda.synchronize()
        _step(ranks, P, C, chunk_heads)          # eager reference on these inputs
        torch.cuda.synchronize()
        want = _outs(ranks)
        for rk in ranks:                         # scribble over the outputs
            for t in (rk.packed, *rk.planes, rk.send, rk.merged):
                t.view(torch.int16).fill_(0x7FC1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outs(ranks)
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {it}: output {i} differs"
