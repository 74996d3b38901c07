"""Bit parity of the HIP path with the CPU oracle on the five workloads at
their full sizes (every element of every stage compared), through the C ABI.

Workloads: tiny round trip (P=2, C=1, 64 tokens/rank, 4 heads of 16);
mid-size (P=2, C=4, 4,096 tokens/rank, 32 heads of 128); the representative
55,413-token shape (P=2, C=4, 27,707 tokens/rank, 56 heads of 128); the same
with Q/K/V read in place from a fused [27,707][21,568] projection output with
64 padding columns and U[-8, 8] values including +-0 and subnormals (its
head merge writes into a padded [27,707][56*128 + 64] output as well); and
P=4, C=4 with 31,000 tokens padded to 31,008.
"""
import numpy as np
import pytest
import torch

import datagen
from datagen import WORKLOADS
from tests.gpu_harness import say
from tests.pipeline import run_pipeline


@pytest.mark.gpu
@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_pipeline_parity(cid, gpu):
    w = WORKLOADS[cid]
    say(f"[cfg{cid}] {w.name}: generating inputs")
    fused = [datagen.fused_source(w, r) for r in range(w.P)]
    merge_layout = {"row_pad": 64} if w.row_pad else {}
    run_pipeline(gpu, w.P, w.C, w.s_local, w.H, w.D, fused, f"cfg{cid}", merge_layout=merge_layout)
    del fused
    torch.cuda.empty_cache()


@pytest.mark.gpu
def test_representative_shape_head_major_attention_side(gpu):
    """The representative shape with the attention side stored head-major
    (BHTD: Q/K/V and O as [G][S][D]): unpack writes it and split reads it."""
    w = WORKLOADS[3]
    fused = [datagen.fused_source(w, r) for r in range(w.P)]
    run_pipeline(gpu, w.P, w.C, w.s_local, w.H, w.D, fused, "cfg3-bhtd",
                 unpack_layout={"head_major": True}, planes=(2,))
    del fused
    torch.cuda.empty_cache()


@pytest.mark.gpu
def test_config4_pad_sentinel_never_copied(gpu):
    """The 64 padding columns of the fused rows hold a sentinel that must not
    reach the packed buffer."""
    import head_relayout_amd as vrl
    from tests.gpu_harness import to_dev
    from tests.pipeline import dev_qkv

    w = WORKLOADS[4]
    f = datagen.fused_source(w, 0)
    assert (f[:, -w.row_pad:] == datagen.PAD_SENTINEL).all()
    assert not (f[:, :-w.row_pad] == datagen.PAD_SENTINEL).any()
    d = to_dev(f, gpu)
    out = torch.empty(vrl.exchange_elems(0, w.P, w.C, w.s_local, w.H, w.D), dtype=torch.bfloat16,
                      device=gpu)
    vrl.qkv_pack(*dev_qkv(d, w.H, w.D), out, w.P, w.C)
    torch.cuda.synchronize()
    assert not bool((out.view(torch.int16) == datagen.PAD_SENTINEL).any())


@pytest.mark.gpu
@pytest.mark.parametrize("layout", ["dense", "head_major"])
def test_offsets_beyond_2_31_elements(gpu, layout):
    """Wire buffers of 2.2e9 elements (4.4 GB per rank): element offsets pass
    2^31, so every address product must be 64-bit.  P=2, C=2, 90,000
    tokens/rank, 64 heads of 128; the whole path against the oracle, with
    token-major or head-major (head-run kernels) attention side and merge
    output."""
    from dataclasses import replace
    w = replace(WORKLOADS[2], name="large offsets", s_local=90000, H=64, total_tokens=180000, C=2)
    assert 3 * w.s_local * w.H * w.D > 2**31
    say(f"[large-{layout}] generating inputs")
    fused = [datagen.fused_source(w, r) for r in range(w.P)]
    lay = {"dense": {}, "head_major": {"head_major": True}}[layout]
    run_pipeline(gpu, w.P, w.C, w.s_local, w.H, w.D, fused, f"large-{layout}", planes=(1,),
                 unpack_layout=lay, merge_layout=lay)
    del fused
    torch.cuda.empty_cache()


@pytest.mark.gpu
@pytest.mark.parametrize("layout", ["dense", "head_major"])
def test_unpack_eight_ranks_full_size(gpu, layout):
    """The representative sequence (55,416 tokens) split over P=8 ranks of
    6,927 tokens, C=4, 56 heads of 128 (head groups of 7): one rank's QKV
    unpack against the oracle, into token-major [S][G][D] or head-major
    [G][S][D] Q/K/V.  With eight ranks every head-major run crosses seven
    rank boundaries, so the unpack's workgroup walk over (chunk, rank, head)
    runs at a realistic size with many token tiles per block."""
    import head_relayout_amd as vrl
    import oracle
    from tests.gpu_harness import assert_bits_equal, to_dev

    P, C, S_l, H, D = 8, 4, 6927, 56, 128
    G, S = H // P, P * S_l
    n_qkv = 3 * S_l * H * D
    say(f"[unpack-p8-{layout}] oracle")
    recv = datagen.values(n_qkv, seed=8, stream=0)
    want = [np.zeros((S, G, D), dtype=np.uint16) for _ in range(3)]
    oracle.qkv_unpack(oracle.dims(P, C, S_l, H, D), recv, *want)
    say(f"[unpack-p8-{layout}] device")
    bf = dict(dtype=torch.bfloat16, device=gpu)
    if layout == "dense":
        outs = [torch.full((S, G, D), 0, **bf) for _ in range(3)]
        views = outs
    else:
        outs = [torch.full((G, S, D), 0, **bf) for _ in range(3)]
        views = [t.transpose(0, 1) for t in outs]
    vrl.qkv_unpack(to_dev(recv, gpu), *views, P, C)
    torch.cuda.synchronize()
    for q in range(3):
        assert_bits_equal(views[q], want[q], f"unpack P=8 {layout} plane {q}")
    del outs, views
    torch.cuda.empty_cache()
