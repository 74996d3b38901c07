"""Pins of the CPU oracle against things other than itself (no GPU).

* brute-force closed-form index maps on tiny shapes with unique-id payloads;
* the same chains written with PyTorch CPU library routines;
* invariants: round trip, exchange involution, the all-gather closed form
  and its independence of the chunk count, window composition, the
  single-permute forms of the equal-chunk case;
* untouched padding of strided output views.
The allocation-screen byte counts printed on the pages are pinned in
test_allocation_screen.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests import index_maps as im
from tests import torch_chains as tc
from tests.helpers import SENTINEL, padded_view, qkv_views, unique_fused, unique_ids

# (P, C, S_l, H, D, row_pad of the fused source)
SHAPES = [
    (2, 1, 64, 4, 16, 0),   # tiny round-trip workload
    (2, 4, 10, 4, 8, 0),    # ragged chunks [3, 3, 2, 2]
    (3, 2, 7, 6, 8, 0),     # three ranks
    (2, 5, 5, 4, 8, 0),     # as many chunks as tokens
    (8, 3, 9, 8, 4, 0),     # eight ranks, one head per group
    (2, 4, 10, 4, 8, 8),    # fused rows padded by 8 elements
    (2, 3, 11, 4, 8, 1),    # fused rows padded by 1 element
    (1, 2, 6, 3, 8, 0),     # one rank
    (4, 4, 12, 8, 2, 3),    # four ranks, tiny head_dim, odd pad
]
IDS = [f"P{s[0]}C{s[1]}S{s[2]}H{s[3]}D{s[4]}pad{s[5]}" for s in SHAPES]


def _dims(P, C, S_l, H, D):
    return oracle.dims(P, C, S_l, H, D)


def _run_pack(P, C, S_l, H, D, pad, window=None):
    fused = unique_fused(P, S_l, H, D, pad)
    d = _dims(P, C, S_l, H, D)
    packs = []
    for r in range(P):
        q, k, v = qkv_views(fused[r], H, D)
        packed = np.full(oracle.exchange_elems(d, 0), SENTINEL, dtype=np.uint16)
        oracle.qkv_pack(d, q, k, v, packed, *(window or (None, None)))
        packs.append(packed)
    return fused, packs


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_pack_matches_index_map(shape):
    P, C, S_l, H, D, pad = shape
    fused, packs = _run_pack(P, C, S_l, H, D, pad)
    for r in range(P):
        expect = im.pack(P, C, S_l, H, D, qkv_views(fused[r], H, D))
        np.testing.assert_array_equal(packs[r], expect)


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
@pytest.mark.parametrize("head_major", [False, True])
def test_unpack_matches_index_map(shape, head_major):
    P, C, S_l, H, D, pad = shape
    G, S = H // P, P * S_l
    d = _dims(P, C, S_l, H, D)
    recv = unique_ids(3 * S_l * H * D)
    got = [padded_view(S, G, D, row_pad=pad, head_major=head_major) for _ in range(3)]
    oracle.qkv_unpack(d, recv, *[g[0] for g in got])
    want = [padded_view(S, G, D, row_pad=pad, head_major=head_major) for _ in range(3)]
    im.unpack(P, C, S_l, H, D, recv, [w[0] for w in want])
    for (gv, gb), (wv, wb) in zip(got, want):
        np.testing.assert_array_equal(gb, wb)        # padding untouched as well


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
@pytest.mark.parametrize("head_major", [False, True])
def test_split_matches_index_map(shape, head_major):
    P, C, S_l, H, D, pad = shape
    G, S = H // P, P * S_l
    d = _dims(P, C, S_l, H, D)
    o, ob = padded_view(S, G, D, row_pad=pad, head_major=head_major)
    o[...] = unique_ids(S * G * D).reshape(S, G, D)
    send = np.full(oracle.exchange_elems(d, 1), SENTINEL, dtype=np.uint16)
    oracle.attn_split(d, o, send)
    np.testing.assert_array_equal(send, im.split(P, C, S_l, H, D, o))


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
@pytest.mark.parametrize("head_major", [False, True])
def test_merge_matches_index_map(shape, head_major):
    P, C, S_l, H, D, pad = shape
    d = _dims(P, C, S_l, H, D)
    recv = unique_ids(S_l * H * D)
    got, gb = padded_view(S_l, H, D, row_pad=pad, head_major=head_major)
    oracle.head_merge(d, recv, got)
    want, wb = padded_view(S_l, H, D, row_pad=pad, head_major=head_major)
    im.merge(P, C, S_l, H, D, recv, want)
    np.testing.assert_array_equal(gb, wb)


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
@pytest.mark.parametrize("which", [0, 1])
def test_exchange_matches_index_map_and_is_involution(shape, which):
    P, C, S_l, H, D, _ = shape
    d = _dims(P, C, S_l, H, D)
    n = oracle.exchange_elems(d, which)
    sends = [unique_ids(n, base=r * n) if P * n <= 0x10000 else
             np.random.default_rng(r).integers(0, 0x10000, n, dtype=np.uint16) for r in range(P)]
    recvs = [np.zeros(n, dtype=np.uint16) for _ in range(P)]
    oracle.exchange(d, which, sends, recvs)
    want = im.exchange(P, C, S_l, H, D, which, sends)
    for g, w in zip(recvs, want):
        np.testing.assert_array_equal(g, w)
    back = [np.zeros(n, dtype=np.uint16) for _ in range(P)]
    oracle.exchange(d, which, recvs, back)
    for b, s in zip(back, sends):
        np.testing.assert_array_equal(b, s)


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_windows_compose_to_full_call(shape):
    """Each single-chunk window writes only its own blocks / rows, and the
    windows together give the full call."""
    P, C, S_l, H, D, pad = shape
    G, S = H // P, P * S_l
    d = _dims(P, C, S_l, H, D)
    fused = unique_fused(P, S_l, H, D, pad)
    q, k, v = qkv_views(fused[0], H, D)
    full = np.full(oracle.exchange_elems(d, 0), SENTINEL, dtype=np.uint16)
    oracle.qkv_pack(d, q, k, v, full)
    acc = np.full_like(full, SENTINEL)
    for c in range(C):
        one = np.full_like(full, SENTINEL)
        oracle.qkv_pack(d, q, k, v, one, c, c + 1)
        np.testing.assert_array_equal(one, im.pack(P, C, S_l, H, D, (q, k, v), window=(c, c + 1),
                                                   out=np.full_like(full, SENTINEL)))
        oracle.qkv_pack(d, q, k, v, acc, c, c + 1)
    np.testing.assert_array_equal(acc, full)

    recv = full
    outs_full = [padded_view(S, G, D) for _ in range(3)]
    oracle.qkv_unpack(d, recv, *[o[0] for o in outs_full])
    outs_acc = [padded_view(S, G, D) for _ in range(3)]
    for c in range(C):
        oracle.qkv_unpack(d, recv, *[o[0] for o in outs_acc], c, c + 1)
    for a, b in zip(outs_acc, outs_full):
        np.testing.assert_array_equal(a[1], b[1])

    o = outs_full[0][0]
    send_full = np.full(oracle.exchange_elems(d, 1), SENTINEL, dtype=np.uint16)
    oracle.attn_split(d, o, send_full)
    send_acc = np.full_like(send_full, SENTINEL)
    for c in range(C):
        oracle.attn_split(d, o, send_acc, c, c + 1)
    np.testing.assert_array_equal(send_acc, send_full)

    m_full, mb_full = padded_view(S_l, H, D, row_pad=pad)
    oracle.head_merge(d, send_full, m_full)
    m_acc, mb_acc = padded_view(S_l, H, D, row_pad=pad)
    for c in range(C):
        oracle.head_merge(d, send_full, m_acc, c, c + 1)
        w, wb = padded_view(S_l, H, D, row_pad=pad)
        im.merge(P, C, S_l, H, D, send_full, w, window=(c, c + 1))
        one, oneb = padded_view(S_l, H, D, row_pad=pad)
        oracle.head_merge(d, send_full, one, c, c + 1)
        np.testing.assert_array_equal(oneb, wb)
    np.testing.assert_array_equal(mb_acc, mb_full)


def _t(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16))


@pytest.mark.parametrize("shape", SHAPES + [(2, 4, 4096, 32, 128, 0)],
                         ids=IDS + ["mid-size P2C4S4096H32D128"])
def test_chains_match_torch_cpu(shape):
    P, C, S_l, H, D, pad = shape
    G, S = H // P, P * S_l
    d = _dims(P, C, S_l, H, D)
    rng = np.random.default_rng(1234)
    fused = rng.integers(0, 0x10000, size=(S_l, 3 * H * D + pad), dtype=np.uint16)
    q, k, v = qkv_views(fused, H, D)
    packed = np.zeros(oracle.exchange_elems(d, 0), dtype=np.uint16)
    oracle.qkv_pack(d, q, k, v, packed)
    ref = tc.pack(P, C, S_l, H, D, _t(q), _t(k), _t(v))
    np.testing.assert_array_equal(packed.view(np.int16), ref.numpy())

    outs = [np.zeros((S, G, D), dtype=np.uint16) for _ in range(3)]
    oracle.qkv_unpack(d, packed, *outs)
    for o, r in zip(outs, tc.unpack(P, C, S_l, H, D, _t(packed))):
        np.testing.assert_array_equal(o.view(np.int16), r.numpy())

    send = np.zeros(oracle.exchange_elems(d, 1), dtype=np.uint16)
    oracle.attn_split(d, outs[1], send)
    np.testing.assert_array_equal(send.view(np.int16), tc.split(P, C, S_l, H, D, _t(outs[1])).numpy())

    merged = np.zeros((S_l, H, D), dtype=np.uint16)
    oracle.head_merge(d, send, merged)
    np.testing.assert_array_equal(merged.view(np.int16), tc.merge(P, C, S_l, H, D, _t(send)).numpy())


@pytest.mark.parametrize("shape", [s for s in SHAPES if s[2] % s[1] == 0],
                         ids=[i for s, i in zip(SHAPES, IDS) if s[2] % s[1] == 0])
def test_single_permute_forms(shape):
    """With equal chunks the per-block chains equal one view/permute/contiguous."""
    P, C, S_l, H, D, pad = shape
    G, S = H // P, P * S_l
    d = _dims(P, C, S_l, H, D)
    fused = unique_fused(P, S_l, H, D, pad)
    q, k, v = qkv_views(fused[0], H, D)
    a = np.zeros(oracle.exchange_elems(d, 0), dtype=np.uint16)
    b = np.ones_like(a)
    oracle.qkv_pack(d, q, k, v, a)
    oracle.qkv_pack_permute(d, q, k, v, b)
    np.testing.assert_array_equal(a, b)
    ua = [np.zeros((S, G, D), dtype=np.uint16) for _ in range(3)]
    ub = [np.ones((S, G, D), dtype=np.uint16) for _ in range(3)]
    oracle.qkv_unpack(d, a, *ua)
    oracle.qkv_unpack_permute(d, a, *ub)
    for x, y in zip(ua, ub):
        np.testing.assert_array_equal(x, y)


def _round_trip(P, C, S_l, H, D, fused):
    """pack -> exchange -> unpack -> split(O := plane q) -> exchange -> merge,
    for q = 0, 1, 2.  Returns (unpacked planes per rank, merged per q per rank)."""
    G, S = H // P, P * S_l
    d = _dims(P, C, S_l, H, D)
    packs = []
    for r in range(P):
        packed = np.zeros(oracle.exchange_elems(d, 0), dtype=np.uint16)
        oracle.qkv_pack(d, *qkv_views(fused[r], H, D), packed)
        packs.append(packed)
    recvs = [np.zeros_like(p) for p in packs]
    oracle.exchange(d, 0, packs, recvs)
    planes = []
    for r in range(P):
        outs = [np.zeros((S, G, D), dtype=np.uint16) for _ in range(3)]
        oracle.qkv_unpack(d, recvs[r], *outs)
        planes.append(outs)
    merged = []
    for qi in range(3):
        sends = []
        for r in range(P):
            send = np.zeros(oracle.exchange_elems(d, 1), dtype=np.uint16)
            oracle.attn_split(d, planes[r][qi], send)
            sends.append(send)
        back = [np.zeros_like(s) for s in sends]
        oracle.exchange(d, 1, sends, back)
        outs = []
        for r in range(P):
            m = np.zeros((S_l, H, D), dtype=np.uint16)
            oracle.head_merge(d, back[r], m)
            outs.append(m)
        merged.append(outs)
    return planes, merged


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_round_trip_identity(shape):
    P, C, S_l, H, D, pad = shape
    fused = unique_fused(P, S_l, H, D, pad)
    _, merged = _round_trip(P, C, S_l, H, D, fused)
    for qi in range(3):
        for r in range(P):
            np.testing.assert_array_equal(merged[qi][r], qkv_views(fused[r], H, D)[qi])


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_allgather_closed_form_independent_of_chunks(shape):
    """unpack(exchange(pack(x))) on rank r is the all-gather of head group r
    along tokens: X_q[s*S_l + tau][g] = src_{s,q}[tau][r*G + g], for any C."""
    P, C, S_l, H, D, pad = shape
    G = H // P
    fused = unique_fused(P, S_l, H, D, pad)
    for CC in sorted({1, C, S_l}):
        planes, _ = _round_trip(P, CC, S_l, H, D, fused)
        for r in range(P):
            for qi in range(3):
                want = np.concatenate(
                    [qkv_views(fused[s], H, D)[qi][:, r * G:(r + 1) * G, :] for s in range(P)], 0)
                np.testing.assert_array_equal(planes[r][qi], want)


def test_oracle_rejects_bad_dims():
    q = np.zeros((4, 4, 8), dtype=np.uint16)
    packed = np.zeros(3 * 4 * 4 * 8, dtype=np.uint16)
    for bad in [(3, 1, 4, 4, 8), (2, 5, 4, 4, 8), (0, 1, 4, 4, 8), (2, 1, 4, 4, 0)]:
        with pytest.raises(ValueError):
            oracle.qkv_pack(oracle.dims(*bad), q, q, q, packed)
    with pytest.raises(ValueError):
        oracle.qkv_pack(oracle.dims(2, 2, 4, 4, 8), q, q, q, packed, 1, 1)
