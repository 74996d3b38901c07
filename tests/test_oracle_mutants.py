"""Plants plausible mistakes in copies of the oracle and checks that the pins
catch every one of them (no GPU).

Each mutant is one textual edit of oracle/oracle.c (a dropped term, a wrong
index, a transposed operand, a wrong chunk rule), compiled with gcc into a
temporary directory and run against a compact set of the pins: brute-force
index maps, exchange map, round trip, the all-gather closed form and window
composition.  Every mutant keeps all accesses in bounds.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import index_maps as im
from tests.helpers import SENTINEL, padded_view, qkv_views, unique_fused, unique_ids
from tests.test_oracle import _round_trip

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "pack drops the chunk offset":
        ("tv_narrow(Xv, 1, chunk_start(d, c) - t0, T)", "tv_narrow(Xv, 1, 0, T)"),
    "pack reads the wrong dest group":
        ("tv_narrow(Xv, 1, chunk_start(d, c) - t0, T), 2, dd)",
         "tv_narrow(Xv, 1, chunk_start(d, c) - t0, T), 2, d->P - 1 - dd)"),
    "pack takes K for Q":
        ("view3(q, d->s_local, d->H, D), 0, t0, n)", "view3(k, d->s_local, d->H, D), 0, t0, n)"),
    "extra tokens go to the last chunks":
        ("return base + (c < extra ? 1 : 0);", "return base + (c >= d->C - extra ? 1 : 0);"),
    "pack window ignores its first token":
        ("t0 = chunk_start(d, c_begin), n = chunk_start(d, c_end) - t0;\n    tv src[3]",
         "t0 = 0 * chunk_start(d, c_begin), n = chunk_start(d, c_end) - chunk_start(d, c_begin);\n"
         "    tv src[3]"),
    "unpack drops the source-rank token offset":
        ("tv_narrow(out, 0, s * d->s_local + chunk_start(d, c), T)",
         "tv_narrow(out, 0, chunk_start(d, c), T)"),
    "unpack reads the wrong plane":
        ("parts[i++] = tv_select(blk, 0, qi);", "parts[i++] = tv_select(blk, 0, (qi + 1) % 3);"),
    "split always reads rank 0's tokens":
        ("tv_narrow(tv_select(Ov, 0, dd), 0, chunk_start(d, c), T)",
         "tv_narrow(tv_select(Ov, 0, 0), 0, chunk_start(d, c), T)"),
    "merge reverses the source groups":
        ("wire_block_start(d, s, c_begin, G * D), 3, bs);",
         "wire_block_start(d, d->P - 1 - s, c_begin, G * D), 3, bs);"),
    "exchange transposes sender and receiver blocks":
        ("tv_dense(send[s] + wire_block_start(d, r, c, per_token), 1, sz)",
         "tv_dense(send[s] + wire_block_start(d, s, c, per_token), 1, sz)"),
}

PIN_SHAPES = [(2, 4, 10, 4, 8, 0), (3, 2, 7, 6, 8, 3)]


def _pins_hold() -> bool:
    """True when every compact pin passes for the oracle build in use."""
    try:
        for P, C, S_l, H, D, pad in PIN_SHAPES:
            G, S = H // P, P * S_l
            d = oracle.dims(P, C, S_l, H, D)
            fused = unique_fused(P, S_l, H, D, pad)
            q, k, v = qkv_views(fused[0], H, D)
            packed = np.full(oracle.exchange_elems(d, 0), SENTINEL, dtype=np.uint16)
            oracle.qkv_pack(d, q, k, v, packed)
            np.testing.assert_array_equal(packed, im.pack(P, C, S_l, H, D, (q, k, v)))
            for c in range(C):
                one = np.full_like(packed, SENTINEL)
                oracle.qkv_pack(d, q, k, v, one, c, c + 1)
                want = im.pack(P, C, S_l, H, D, (q, k, v), (c, c + 1), np.full_like(packed, SENTINEL))
                np.testing.assert_array_equal(one, want)

            recv = unique_ids(3 * S_l * H * D)
            got = [padded_view(S, G, D) for _ in range(3)]
            oracle.qkv_unpack(d, recv, *[g[0] for g in got])
            want = [padded_view(S, G, D) for _ in range(3)]
            im.unpack(P, C, S_l, H, D, recv, [w[0] for w in want])
            for a, b in zip(got, want):
                np.testing.assert_array_equal(a[1], b[1])

            o = got[1][0]
            send = np.full(oracle.exchange_elems(d, 1), SENTINEL, dtype=np.uint16)
            oracle.attn_split(d, o, send)
            np.testing.assert_array_equal(send, im.split(P, C, S_l, H, D, o))

            m, mb = padded_view(S_l, H, D, row_pad=pad)
            oracle.head_merge(d, send, m)
            w, wb = padded_view(S_l, H, D, row_pad=pad)
            im.merge(P, C, S_l, H, D, send, w)
            np.testing.assert_array_equal(mb, wb)

            sends = [unique_ids(S_l * H * D, base=r * S_l * H * D) for r in range(P)]
            recvs = [np.zeros_like(x) for x in sends]
            oracle.exchange(d, 1, sends, recvs)
            for a, b in zip(recvs, im.exchange(P, C, S_l, H, D, 1, sends)):
                np.testing.assert_array_equal(a, b)

            planes, merged = _round_trip(P, C, S_l, H, D, fused)
            for qi in range(3):
                for r in range(P):
                    np.testing.assert_array_equal(merged[qi][r], qkv_views(fused[r], H, D)[qi])
                    want = np.concatenate(
                        [qkv_views(fused[s], H, D)[qi][:, r * G:(r + 1) * G] for s in range(P)], 0)
                    np.testing.assert_array_equal(planes[r][qi], want)
    except AssertionError:
        return False
    return True


def test_pins_hold_for_the_oracle():
    assert _pins_hold()


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", "-o",
                           str(so), str(mutated)])
    with oracle.library(str(so)):
        assert not _pins_hold(), f"no pin caught the mutant: {name}"


# ---- head-chunked chains -------------------------------------------------------

MUTANTS_HC = {
    "head-chunk pack reverses the chunks":
        ("tv_select(tv_select(Xv, 2, dd), 2, c)", "tv_select(tv_select(Xv, 2, dd), 2, d->C - 1 - c)"),
    "head-chunk unpack writes every window at head 0":
        ("tv_narrow(view3(outs[qi], S, G, D), 1, c_begin * Gc, W * Gc)",
         "tv_narrow(view3(outs[qi], S, G, D), 1, 0, W * Gc)"),
    "head-chunk split always reads chunk 0":
        ("tv_select(tv_select(Ov, 0, dd), 1, c)", "tv_select(tv_select(Ov, 0, dd), 1, 0)"),
    "head-chunk merge reverses the sources":
        ("hc_block_start(d, s, c_begin, S_l * Gc * D), 4, bs)",
         "hc_block_start(d, d->P - 1 - s, c_begin, S_l * Gc * D), 4, bs)"),
}

HC_PIN_SHAPES = [(2, 2, 6, 8, 8, 0), (3, 2, 5, 12, 8, 1)]


def _hc_pins_hold() -> bool:
    HC = dict(chunk_heads=True)
    try:
        for P, C, S_l, H, D, pad in HC_PIN_SHAPES:
            G, S = H // P, P * S_l
            d = oracle.dims(P, C, S_l, H, D)
            q, k, v = qkv_views(unique_fused(1, S_l, H, D, pad)[0], H, D)
            packed = np.full(oracle.exchange_elems(d, 0), SENTINEL, dtype=np.uint16)
            oracle.qkv_pack(d, q, k, v, packed, **HC)
            np.testing.assert_array_equal(packed, im.pack_hc(P, C, S_l, H, D, (q, k, v)))
            recv = unique_ids(3 * S_l * H * D)
            for c in range(C):
                got = [padded_view(S, G, D) for _ in range(3)]
                oracle.qkv_unpack(d, recv, *[g[0] for g in got], c, c + 1, **HC)
                want = [padded_view(S, G, D) for _ in range(3)]
                im.unpack_hc(P, C, S_l, H, D, recv, [w[0] for w in want], (c, c + 1))
                for a, b in zip(got, want):
                    np.testing.assert_array_equal(a[1], b[1])
            o = np.ascontiguousarray(unique_ids(S * G * D).reshape(S, G, D))
            send = np.full(oracle.exchange_elems(d, 1), SENTINEL, dtype=np.uint16)
            oracle.attn_split(d, o, send, **HC)
            np.testing.assert_array_equal(send, im.split_hc(P, C, S_l, H, D, o))
            m, mb = padded_view(S_l, H, D, row_pad=pad)
            oracle.head_merge(d, send, m, **HC)
            w, wb = padded_view(S_l, H, D, row_pad=pad)
            im.merge_hc(P, C, S_l, H, D, send, w)
            np.testing.assert_array_equal(mb, wb)
    except AssertionError:
        return False
    return True


def test_head_chunk_pins_hold_for_the_oracle():
    assert _hc_pins_hold()


@pytest.mark.parametrize("name", list(MUTANTS_HC))
def test_head_chunk_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS_HC[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", "-o",
                           str(so), str(mutated)])
    with oracle.library(str(so)):
        assert not _hc_pins_hold(), f"no pin caught the mutant: {name}"
