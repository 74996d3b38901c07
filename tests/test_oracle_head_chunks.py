"""Pins of the oracle's head-chunked chains (no GPU).

The other reading of the four-chunk layout splits each destination's head
group into C chunks of Gc = G / C heads instead of splitting tokens.  Pinned
like the token-chunked chains: closed-form index maps on tiny shapes with
unique ids, the chains in torch CPU routines, the exchange map and its
involution, window composition, the round trip; and against the
token-chunked chains themselves: unpack(exchange(pack(x))) is the same
all-gather of head group r under either reading, and with C = 1 the two
wire layouts are one and the same.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests import index_maps as im
from tests import torch_chains as tc
from tests.helpers import SENTINEL, padded_view, qkv_views, unique_fused, unique_ids

# (P, C, S_l, H, D, source row pad); every G = H / P divisible by C
SHAPES = [
    (2, 2, 10, 8, 8, 0),
    (2, 4, 10, 8, 8, 0),     # one head per chunk
    (3, 2, 7, 12, 8, 3),
    (4, 2, 6, 16, 4, 0),
    (1, 3, 5, 6, 8, 1),
    (2, 1, 64, 4, 16, 0),    # C = 1
    (2, 4, 3, 8, 8, 0),      # more chunks than tokens
]
IDS = [f"P{s[0]}C{s[1]}S{s[2]}H{s[3]}D{s[4]}pad{s[5]}" for s in SHAPES]
HC = dict(chunk_heads=True)


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_pack_matches_index_map(shape):
    P, C, S_l, H, D, pad = shape
    d = oracle.dims(P, C, S_l, H, D)
    for f in unique_fused(P, S_l, H, D, pad):
        packed = np.full(oracle.exchange_elems(d, 0), SENTINEL, dtype=np.uint16)
        oracle.qkv_pack(d, *qkv_views(f, H, D), packed, **HC)
        np.testing.assert_array_equal(packed, im.pack_hc(P, C, S_l, H, D, qkv_views(f, H, D)))


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
@pytest.mark.parametrize("head_major", [False, True])
def test_unpack_split_merge_match_index_maps(shape, head_major):
    P, C, S_l, H, D, pad = shape
    G, S = H // P, P * S_l
    d = oracle.dims(P, C, S_l, H, D)
    recv = unique_ids(3 * S_l * H * D)
    got = [padded_view(S, G, D, row_pad=pad, head_major=head_major) for _ in range(3)]
    oracle.qkv_unpack(d, recv, *[g[0] for g in got], **HC)
    want = [padded_view(S, G, D, row_pad=pad, head_major=head_major) for _ in range(3)]
    im.unpack_hc(P, C, S_l, H, D, recv, [w[0] for w in want])
    for a, b in zip(got, want):
        np.testing.assert_array_equal(a[1], b[1])

    o = got[2][0]
    send = np.full(oracle.exchange_elems(d, 1), SENTINEL, dtype=np.uint16)
    oracle.attn_split(d, o, send, **HC)
    np.testing.assert_array_equal(send, im.split_hc(P, C, S_l, H, D, o))

    m, mb = padded_view(S_l, H, D, row_pad=pad, head_major=head_major)
    oracle.head_merge(d, send, m, **HC)
    w, wb = padded_view(S_l, H, D, row_pad=pad, head_major=head_major)
    im.merge_hc(P, C, S_l, H, D, send, w)
    np.testing.assert_array_equal(mb, wb)


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
@pytest.mark.parametrize("which", [0, 1])
def test_exchange_map_and_involution(shape, which):
    P, C, S_l, H, D, _ = shape
    d = oracle.dims(P, C, S_l, H, D)
    n = oracle.exchange_elems(d, which)
    sends = [np.random.default_rng(r).integers(0, 0x10000, n, dtype=np.uint16) for r in range(P)]
    recvs = [np.zeros(n, dtype=np.uint16) for _ in range(P)]
    oracle.exchange(d, which, sends, recvs, **HC)
    for g, w in zip(recvs, im.exchange_hc(P, C, S_l, H, D, which, sends)):
        np.testing.assert_array_equal(g, w)
    back = [np.zeros(n, dtype=np.uint16) for _ in range(P)]
    oracle.exchange(d, which, recvs, back, **HC)
    for b, s in zip(back, sends):
        np.testing.assert_array_equal(b, s)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16))


@pytest.mark.parametrize("shape", SHAPES + [(2, 4, 4096, 32, 128, 0)], ids=IDS + ["mid-size"])
def test_chains_match_torch_cpu(shape):
    P, C, S_l, H, D, pad = shape
    G, S = H // P, P * S_l
    d = oracle.dims(P, C, S_l, H, D)
    fused = np.random.default_rng(99).integers(0, 0x10000, size=(S_l, 3 * H * D + pad), dtype=np.uint16)
    q, k, v = qkv_views(fused, H, D)
    packed = np.zeros(oracle.exchange_elems(d, 0), dtype=np.uint16)
    oracle.qkv_pack(d, q, k, v, packed, **HC)
    np.testing.assert_array_equal(packed.view(np.int16), tc.pack_hc(P, C, S_l, H, D, _t(q), _t(k), _t(v)).numpy())
    outs = [np.zeros((S, G, D), dtype=np.uint16) for _ in range(3)]
    oracle.qkv_unpack(d, packed, *outs, **HC)
    for o, r in zip(outs, tc.unpack_hc(P, C, S_l, H, D, _t(packed))):
        np.testing.assert_array_equal(o.view(np.int16), r.numpy())
    send = np.zeros(oracle.exchange_elems(d, 1), dtype=np.uint16)
    oracle.attn_split(d, outs[0], send, **HC)
    np.testing.assert_array_equal(send.view(np.int16), tc.split_hc(P, C, S_l, H, D, _t(outs[0])).numpy())
    merged = np.zeros((S_l, H, D), dtype=np.uint16)
    oracle.head_merge(d, send, merged, **HC)
    np.testing.assert_array_equal(merged.view(np.int16), tc.merge_hc(P, C, S_l, H, D, _t(send)).numpy())


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_windows_compose(shape):
    P, C, S_l, H, D, pad = shape
    G, S = H // P, P * S_l
    d = oracle.dims(P, C, S_l, H, D)
    q, k, v = qkv_views(unique_fused(1, S_l, H, D, pad)[0], H, D)
    full = np.full(oracle.exchange_elems(d, 0), SENTINEL, dtype=np.uint16)
    oracle.qkv_pack(d, q, k, v, full, **HC)
    acc = np.full_like(full, SENTINEL)
    for c in range(C):
        one = np.full_like(full, SENTINEL)
        oracle.qkv_pack(d, q, k, v, one, c, c + 1, **HC)
        want = im.pack_hc(P, C, S_l, H, D, (q, k, v), (c, c + 1), np.full_like(full, SENTINEL))
        np.testing.assert_array_equal(one, want)
        oracle.qkv_pack(d, q, k, v, acc, c, c + 1, **HC)
    np.testing.assert_array_equal(acc, full)
    fo = [padded_view(S, G, D) for _ in range(3)]
    oracle.qkv_unpack(d, full, *[x[0] for x in fo], **HC)
    ao = [padded_view(S, G, D) for _ in range(3)]
    for c in range(C):
        oracle.qkv_unpack(d, full, *[x[0] for x in ao], c, c + 1, **HC)
    for a, b in zip(ao, fo):
        np.testing.assert_array_equal(a[1], b[1])
    send = np.full(oracle.exchange_elems(d, 1), SENTINEL, dtype=np.uint16)
    oracle.attn_split(d, fo[0][0], send, **HC)
    sacc = np.full_like(send, SENTINEL)
    for c in range(C):
        oracle.attn_split(d, fo[0][0], sacc, c, c + 1, **HC)
    np.testing.assert_array_equal(sacc, send)
    m, mb = padded_view(S_l, H, D, row_pad=pad)
    oracle.head_merge(d, send, m, **HC)
    ma, mab = padded_view(S_l, H, D, row_pad=pad)
    for c in range(C):
        oracle.head_merge(d, send, ma, c, c + 1, **HC)
    np.testing.assert_array_equal(mab, mb)


def _path(P, C, S_l, H, D, fused, chunk_heads):
    G, S = H // P, P * S_l
    d = oracle.dims(P, C, S_l, H, D)
    kw = dict(chunk_heads=chunk_heads)
    packs = []
    for f in fused:
        p = np.zeros(oracle.exchange_elems(d, 0), dtype=np.uint16)
        oracle.qkv_pack(d, *qkv_views(f, H, D), p, **kw)
        packs.append(p)
    recvs = [np.zeros_like(p) for p in packs]
    oracle.exchange(d, 0, packs, recvs, **kw)
    planes = []
    for r in range(P):
        outs = [np.zeros((S, G, D), dtype=np.uint16) for _ in range(3)]
        oracle.qkv_unpack(d, recvs[r], *outs, **kw)
        planes.append(outs)
    merged = []
    for qi in range(3):
        sends = []
        for r in range(P):
            s = np.zeros(oracle.exchange_elems(d, 1), dtype=np.uint16)
            oracle.attn_split(d, planes[r][qi], s, **kw)
            sends.append(s)
        backs = [np.zeros_like(s) for s in sends]
        oracle.exchange(d, 1, sends, backs, **kw)
        row = []
        for r in range(P):
            m = np.zeros((S_l, H, D), dtype=np.uint16)
            oracle.head_merge(d, backs[r], m, **kw)
            row.append(m)
        merged.append(row)
    return packs, planes, merged


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_round_trip_and_agreement_with_token_chunks(shape):
    P, C, S_l, H, D, pad = shape
    fused = unique_fused(P, S_l, H, D, pad)
    packs_h, planes_h, merged_h = _path(P, C, S_l, H, D, fused, True)
    for qi in range(3):
        for r in range(P):
            np.testing.assert_array_equal(merged_h[qi][r], qkv_views(fused[r], H, D)[qi])
    # the attention side does not depend on which axis the chunks split
    Ct = min(C, S_l)
    packs_t, planes_t, _ = _path(P, Ct, S_l, H, D, fused, False)
    for r in range(P):
        for qi in range(3):
            np.testing.assert_array_equal(planes_h[r][qi], planes_t[r][qi])
    if C == 1:
        for a, b in zip(packs_h, packs_t):
            np.testing.assert_array_equal(a, b)


def test_rejects_head_groups_not_divisible_by_chunks():
    q = np.zeros((4, 6, 8), dtype=np.uint16)
    packed = np.zeros(3 * 4 * 6 * 8, dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.qkv_pack(oracle.dims(2, 2, 4, 6, 8), q, q, q, packed, **HC)   # G = 3, C = 2
