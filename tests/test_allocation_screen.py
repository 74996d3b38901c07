"""Pins the oracle's chains to the allocation screen printed on the pages.

At the representative shape the materialised pack and merge chains peak at
exactly twice their outputs (two materialisations), the direct outputs are
1,191,622,656 B and 397,207,552 B, and a one-chunk split window keeps a
94.7 MiB output (fixture: tests/golden/allocation_screen.txt, with its
citation).  The chains run on uninitialised buffers: their peak does not
depend on the values.
"""
import numpy as np

import oracle
from datagen import WORKLOADS
from tests.golden.load import load
from tests.helpers import qkv_views


def test_allocation_screen_matches_pages():
    g = load("allocation_screen.txt")
    w = WORKLOADS[3]
    d = oracle.dims(**w.dims())

    fused = np.empty((w.s_local, w.row_stride), dtype=np.uint16)
    packed = np.empty(oracle.exchange_elems(d, 0), dtype=np.uint16)
    peak = oracle.qkv_pack(d, *qkv_views(fused, w.H, w.D), packed)
    assert packed.nbytes == g["pack_direct_peak_bytes"]
    assert peak == g["pack_reference_peak_bytes"]
    assert round((peak - packed.nbytes) / 2**20, 1) == g["pack_saving_mib"]
    assert round(100 * (peak - packed.nbytes) / peak) == g["pack_saving_percent"]
    del fused, packed

    recv = np.empty(oracle.exchange_elems(d, 1), dtype=np.uint16)
    out = np.empty((w.s_local, w.H, w.D), dtype=np.uint16)
    peak = oracle.head_merge(d, recv, out)
    assert out.nbytes == g["merge_direct_peak_bytes"]
    assert peak == g["merge_reference_peak_bytes"]
    assert round((peak - out.nbytes) / 2**20, 1) == g["merge_saving_mib"]
    assert round(100 * (peak - out.nbytes) / peak) == g["merge_saving_percent"]
    del out

    o = np.empty((w.S, w.G, w.D), dtype=np.uint16)
    for c in range(w.C):
        peak = oracle.attn_split(d, o, recv, c, c + 1)
        assert round(peak / 2**20, 1) == g["split_output_mib"]


def test_allocation_screen_head_chunk_reading():
    """The same screen under the head-chunk reading of the four-chunk layout
    (chunks split each head group): pack and merge peaks are unchanged, and
    a one-chunk split window (all tokens, 7 of 28 heads) also rounds to the
    page's 94.7 MiB, which is why that figure cannot decide the reading."""
    g = load("allocation_screen.txt")
    w = WORKLOADS[3]
    d = oracle.dims(**w.dims())
    hc = dict(chunk_heads=True)

    fused = np.empty((w.s_local, w.row_stride), dtype=np.uint16)
    packed = np.empty(oracle.exchange_elems(d, 0), dtype=np.uint16)
    assert oracle.qkv_pack(d, *qkv_views(fused, w.H, w.D), packed, **hc) == g["pack_reference_peak_bytes"]
    del fused, packed

    recv = np.empty(oracle.exchange_elems(d, 1), dtype=np.uint16)
    out = np.empty((w.s_local, w.H, w.D), dtype=np.uint16)
    assert oracle.head_merge(d, recv, out, **hc) == g["merge_reference_peak_bytes"]
    del out

    o = np.empty((w.S, w.G, w.D), dtype=np.uint16)
    for c in range(w.C):
        peak = oracle.attn_split(d, o, recv, c, c + 1, **hc)
        assert peak == w.S * (w.G // w.C) * w.D * 2      # 99,301,888 B
        assert round(peak / 2**20, 1) == g["split_output_mib"]
