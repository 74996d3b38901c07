"""Seeded random parity sweep of all four relayouts against the oracle.

Each case draws P (1-6, 8 or 16 ranks), the head-group size (1-6, 8, 12
or 28 heads: the LDS transpose then tiles several heads of a group),
head_dim, tokens per rank,
the chunk reading (tokens or heads) and count, a chunk window, and the
layouts of every operand: the pack's Q/K/V either as column blocks of fused
projection rows (with padded rows) or each in a layout of its own, and the
attention side and merge output in dense, padded-row, padded-head or
head-major layouts; device operands start 0-4 elements into their
allocation.  Every op writes into a sentinel-filled buffer (with guard
bands); the whole buffer, untouched parts included, must equal the oracle's
result on a buffer filled the same way.  Values are random 16-bit patterns
(negative numbers, infinities and NaN payloads included) except the
sentinel itself, so that a skipped write cannot go unseen.
"""
import os

import numpy as np
import pytest
import torch

import head_relayout_amd as vrl
import oracle
from tests.gpu_harness import SENTINEL, assert_bits_equal, assert_guard_intact, say, to_dev

pytestmark = pytest.mark.gpu

# Case count and seed; the environment may ask for a longer or different sweep.
N_CASES = int(os.environ.get("VRL_RANDOM_CASES", "5000"))
SEED = int(os.environ.get("VRL_RANDOM_SEED", "20261202"))


def _layout(rng, rows, heads, D):
    """(shape of a backing buffer, function mapping it to a [rows][heads][D]
    view): dense, padded rows, padded heads (head stride above D) or
    head-major."""
    kind = rng.integers(0, 4)
    if kind == 0:
        return (rows, heads, D), lambda b: b
    if kind == 1:
        pad = int(rng.integers(1, 8))
        return (rows, heads * D + pad), lambda b: b[:, :heads * D].reshape(rows, heads, D) \
            if isinstance(b, np.ndarray) else b[:, :heads * D].unflatten(1, (heads, D))
    if kind == 2:
        pad = int(rng.integers(1, 5))
        return (rows, heads, D + pad), lambda b: b[:, :, :D]
    return (heads, rows, D), lambda b: b.transpose(1, 0, 2) if isinstance(b, np.ndarray) else b.transpose(0, 1)


def _bits(rng, shape):
    """Random 16-bit patterns, none equal to the sentinel."""
    v = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    v[v == SENTINEL] = SENTINEL ^ 1
    return v


def _dev_shifted(host, base, dev):
    """A device copy of `host` starting `base` elements into its allocation."""
    flat = to_dev(np.concatenate([np.zeros(base, np.uint16), host.reshape(-1)]), dev)
    return flat[base:].view(host.shape)


def _sentinel(shape):
    return np.full(shape, SENTINEL, dtype=np.uint16)


def _dev_guarded(host, dev):
    """A device copy of `host` inside an allocation with guard bands."""
    flat = np.concatenate([_sentinel(2048), host.reshape(-1), _sentinel(2048)])
    whole = to_dev(flat, dev)
    return whole[2048:2048 + host.size].view(host.shape), whole


def _case(rng, tokens=(1, 41), dims=(2, 4, 6, 8, 16, 24, 64, 128), max_elems=None):
    while True:
        P = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 16]))
        G = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 28]))
        H = P * G
        D = int(rng.choice(dims))
        S_l = int(rng.integers(*tokens))
        if max_elems is None or 3 * S_l * H * D <= max_elems:
            break
    hc = bool(rng.integers(0, 2))
    if hc:
        C = int(rng.choice([c for c in range(1, G + 1) if G % c == 0]))
    else:
        C = int(rng.integers(1, min(S_l, 6) + 1))
    cb = int(rng.integers(0, C))
    ce = int(rng.integers(cb + 1, C + 1))
    if rng.random() < 0.4:
        cb, ce = 0, C
    return dict(P=P, G=G, H=H, D=D, S_l=S_l, C=C, hc=hc, cb=cb, ce=ce,
                pad=int(rng.choice([0, 0, 1, 2, 3, 8])), base=int(rng.choice([0, 0, 1, 2, 4])),
                fused_src=bool(rng.random() < 0.5))


def test_random_cases(gpu):
    rng = np.random.default_rng(SEED)
    for n in range(N_CASES):
        k = _case(rng)
        if n % 40 == 0:
            say(f"[random] case {n}: {k}")
        _run_case(gpu, rng, k, f"case {n}: {k}")
    say(f"[random] {N_CASES} cases ok")


def test_random_medium_cases(gpu):
    """Forty cases of 100-1,500 tokens per rank and head_dims 16-128 (up to
    six million elements per wire buffer): several token tiles per block and
    per head, so the full-tile paths, the partial last tiles and the head-run
    and LDS-transpose tile walks all run, in every layout."""
    rng = np.random.default_rng(SEED + 1)
    for n in range(40):
        k = _case(rng, tokens=(100, 1501), dims=(16, 32, 64, 128), max_elems=6_000_000)
        say(f"[random medium] case {n}: {k}")
        _run_case(gpu, rng, k, f"medium case {n}: {k}")
    say("[random medium] 40 cases ok")


def _run_case(gpu, rng, k, tag):
    """One case: every op into sentinel-filled, guarded buffers, against the oracle."""
    P, G, H, D, S_l, C, hc, cb, ce = (k[x] for x in ("P", "G", "H", "D", "S_l", "C", "hc", "cb", "ce"))
    S = P * S_l
    kw = dict(chunk_heads=hc)
    od = oracle.dims(P, C, S_l, H, D)
    n_qkv = 3 * S_l * H * D
    n_att = S_l * H * D

    # pack: Q/K/V as column blocks of fused rows with padding, or each plane
    # in a random layout of its own; device copies shifted by `base` elements
    if k.get("fused_src", True):
        fused = _bits(rng, (S_l, 3 * H * D + k["pad"]))
        hq = [fused[:, i * H * D:(i + 1) * H * D].reshape(S_l, H, D) for i in range(3)]
        dfused = _dev_shifted(fused, k["base"], gpu)
        dq = [dfused[:, i * H * D:(i + 1) * H * D].unflatten(1, (H, D)) for i in range(3)]
    else:
        src_lays = [_layout(rng, S_l, H, D) for _ in range(3)]
        bufs = [_bits(rng, shape) for shape, _ in src_lays]
        hq = [f(b) for b, (_, f) in zip(bufs, src_lays)]
        dq = [f(_dev_shifted(b, k["base"], gpu)) for b, (_, f) in zip(bufs, src_lays)]
    want = _sentinel(n_qkv)
    oracle.qkv_pack(od, *hq, want, cb, ce, **kw)
    got, whole = _dev_guarded(_sentinel(n_qkv), gpu)
    vrl.qkv_pack(*dq, got, P, C, cb, ce, **kw)
    torch.cuda.synchronize()
    assert_bits_equal(got, want, f"{tag} pack")
    assert_guard_intact(whole, f"{tag} pack")

    # unpack into random layouts
    recv = _bits(rng, n_qkv)
    drecv = to_dev(recv, gpu)
    lays = [_layout(rng, S, G, D) for _ in range(3)]
    hbufs = [_sentinel(shape) for shape, _ in lays]
    oracle.qkv_unpack(od, recv, *[f(b) for b, (_, f) in zip(hbufs, lays)], cb, ce, **kw)
    dev = [_dev_guarded(_sentinel(shape), gpu) for shape, _ in lays]
    vrl.qkv_unpack(drecv, *[f(d[0]) for d, (_, f) in zip(dev, lays)], P, C, cb, ce, **kw)
    torch.cuda.synchronize()
    for i in range(3):
        assert_bits_equal(dev[i][0], hbufs[i], f"{tag} unpack plane {i}")
        assert_guard_intact(dev[i][1], f"{tag} unpack plane {i}")

    # split from a random layout (the first unpacked plane's buffer, fully
    # overwritten with values first)
    oshape, of = lays[0]
    obuf = _bits(rng, oshape)
    dobuf = to_dev(obuf, gpu)
    want = _sentinel(n_att)
    oracle.attn_split(od, of(obuf), want, cb, ce, **kw)
    got, whole = _dev_guarded(_sentinel(n_att), gpu)
    vrl.attn_split(of(dobuf), got, P, C, cb, ce, **kw)
    torch.cuda.synchronize()
    assert_bits_equal(got, want, f"{tag} split")
    assert_guard_intact(whole, f"{tag} split")

    # merge into a random layout
    back = _bits(rng, n_att)
    mshape, mf = _layout(rng, S_l, H, D)
    hm = _sentinel(mshape)
    oracle.head_merge(od, back, mf(hm), cb, ce, **kw)
    dm, whole = _dev_guarded(_sentinel(mshape), gpu)
    vrl.head_merge(to_dev(back, gpu), mf(dm), P, C, cb, ce, **kw)
    torch.cuda.synchronize()
    assert_bits_equal(dm, hm, f"{tag} merge")
    assert_guard_intact(whole, f"{tag} merge")


@pytest.mark.parametrize("D", [32, 128])
@pytest.mark.parametrize("src", ["head-major", "head-padded"])
def test_pack_from_strided_sources(gpu, src, D):
    """QKV pack from separate Q/K/V that are not rows of a fused projection:
    stored head-major ([H][S_l][D], read through a transposed view; at
    head_dim 32 the LDS transpose, at 128 the direct kernel with general
    head strides) or with padded head rows; two ranks of 1,500 tokens, 56
    heads, four token chunks and then four head chunks, element for element
    against the oracle."""
    rng = np.random.default_rng(SEED + D)
    P, C, S_l, H = 2, 4, 1500, 56
    od = oracle.dims(P, C, S_l, H, D)
    n_qkv = 3 * S_l * H * D
    if src == "head-major":
        bufs = [_bits(rng, (H, S_l, D)) for _ in range(3)]
        hq = [b.transpose(1, 0, 2) for b in bufs]
        dq = [to_dev(b, gpu).transpose(0, 1) for b in bufs]
    else:
        bufs = [_bits(rng, (S_l, H, D + 8)) for _ in range(3)]
        hq = [b[:, :, :D] for b in bufs]
        dq = [to_dev(b, gpu)[:, :, :D] for b in bufs]
    for hc in (False, True):
        say(f"[pack from {src} sources, D={D}, chunk_heads={hc}]")
        want = _sentinel(n_qkv)
        oracle.qkv_pack(od, *hq, want, chunk_heads=hc)
        got, whole = _dev_guarded(_sentinel(n_qkv), gpu)
        vrl.qkv_pack(*dq, got, P, C, chunk_heads=hc)
        torch.cuda.synchronize()
        assert_bits_equal(got, want, f"pack from {src} sources, D={D}, chunk_heads={hc}")
        assert_guard_intact(whole, f"pack from {src} sources, D={D}, chunk_heads={hc}")
