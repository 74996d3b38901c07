"""The head-chunked layout (chunks split each destination's head group) on
the GPU, bit for bit against the oracle's head-chunked chains, through the
C ABI: the five workloads at full size, small shapes with dense, padded and
head-major views, and single-chunk windows."""
import numpy as np
import pytest
import torch

import datagen
import head_relayout_amd as vrl
import oracle
from datagen import WORKLOADS
from tests.gpu_harness import SENTINEL, assert_bits_equal, guarded, say, sentinel_view, to_dev
from tests.pipeline import dev_qkv, host_qkv, run_pipeline
from tests.test_gpu_edges import ids_fused

pytestmark = pytest.mark.gpu
HC = dict(chunk_heads=True)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_pipeline_parity_head_chunks(gpu, cid):
    w = WORKLOADS[cid]
    say(f"[hc cfg{cid}] {w.name}")
    fused = [datagen.fused_source(w, r) for r in range(w.P)]
    run_pipeline(gpu, w.P, w.C, w.s_local, w.H, w.D, fused, f"hc-cfg{cid}",
                 planes=(0,) if cid in (3, 4) else (0, 1, 2), chunk_heads=True)
    del fused
    torch.cuda.empty_cache()


SHAPES = [(2, 2, 10, 8, 8, 0), (2, 4, 10, 8, 8, 0), (3, 2, 7, 12, 8, 3), (4, 2, 6, 16, 4, 0),
          (1, 3, 5, 6, 8, 1), (2, 4, 3, 8, 8, 0), (2, 2, 9, 8, 40, 0), (2, 3, 11, 12, 8, 1)]
IDS = [f"P{s[0]}C{s[1]}S{s[2]}H{s[3]}D{s[4]}pad{s[5]}" for s in SHAPES]


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
@pytest.mark.parametrize("layout", ["dense", "padded", "head_major"])
def test_small_shapes_head_chunks(gpu, shape, layout):
    P, C, S_l, H, D, pad = shape
    lay = {"dense": {}, "padded": {"row_pad": 5}, "head_major": {"head_major": True}}[layout]
    run_pipeline(gpu, P, C, S_l, H, D, ids_fused(P, S_l, H, D, pad),
                 f"hc-{IDS[SHAPES.index(shape)]}-{layout}", unpack_layout=lay, merge_layout=lay,
                 chunk_heads=True)


@pytest.mark.parametrize("cid", [2, 5])
def test_windows_head_chunks(gpu, cid):
    w = WORKLOADS[cid]
    P, C, S_l, H, D, G, S = w.P, w.C, w.s_local, w.H, w.D, w.G, w.S
    od = oracle.dims(P, C, S_l, H, D)
    fused = datagen.fused_source(w, 0)
    dq = dev_qkv(to_dev(fused, gpu), H, D)
    n = vrl.exchange_elems(0, P, C, S_l, H, D, **HC)
    acc, _ = guarded(n, gpu)
    for c in range(C):
        vrl.qkv_pack(*dq, acc, P, C, c, c + 1, **HC)
        ref = np.full(n, SENTINEL, dtype=np.uint16)
        for cc in range(c + 1):
            oracle.qkv_pack(od, *host_qkv(fused, H, D), ref, cc, cc + 1, **HC)
        torch.cuda.synchronize()
        assert_bits_equal(acc, ref, f"hc windows cfg{cid} pack after chunk {c}")
    full = np.zeros(n, dtype=np.uint16)
    oracle.qkv_pack(od, *host_qkv(fused, H, D), full, **HC)
    outs = [sentinel_view(S, G, D, gpu) for _ in range(3)]
    for c in range(C):
        vrl.qkv_unpack(acc, *[o[0] for o in outs], P, C, c, c + 1, **HC)
        ref = [np.full((S, G, D), SENTINEL, dtype=np.uint16) for _ in range(3)]
        for cc in range(c + 1):
            oracle.qkv_unpack(od, full, *ref, cc, cc + 1, **HC)
        torch.cuda.synchronize()
        for i in range(3):
            assert_bits_equal(outs[i][0], ref[i], f"hc windows cfg{cid} unpack after chunk {c} plane {i}")
    o_ref = np.zeros((S, G, D), dtype=np.uint16)
    oracle.qkv_unpack(od, full, o_ref, np.zeros_like(o_ref), np.zeros_like(o_ref), **HC)
    na = vrl.exchange_elems(1, P, C, S_l, H, D, **HC)
    send, _ = guarded(na, gpu)
    out, _ = sentinel_view(S_l, H, D, gpu, row_pad=3)
    ref_send = np.zeros(na, dtype=np.uint16)
    oracle.attn_split(od, o_ref, ref_send, **HC)
    for c in range(C):
        vrl.attn_split(outs[0][0], send, P, C, c, c + 1, **HC)
        vrl.head_merge(send, out, P, C, c, c + 1, **HC)
        rs = np.full(na, SENTINEL, dtype=np.uint16)
        rm = np.full((S_l, H, D), SENTINEL, dtype=np.uint16)
        for cc in range(c + 1):
            oracle.attn_split(od, o_ref, rs, cc, cc + 1, **HC)
            oracle.head_merge(od, ref_send, rm, cc, cc + 1, **HC)
        torch.cuda.synchronize()
        assert_bits_equal(send, rs, f"hc windows cfg{cid} split after chunk {c}")
        assert_bits_equal(out, rm, f"hc windows cfg{cid} merge after chunk {c}")
