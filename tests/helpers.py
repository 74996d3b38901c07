"""Shared test helpers: tiny unique-id inputs and strided numpy views."""
from __future__ import annotations

import numpy as np

SENTINEL = 0x7FC1


def qkv_views(fused: np.ndarray, H: int, D: int):
    """Q, K, V views [S_l][H][D] of a fused [S_l][3*H*D + pad] row buffer."""
    S_l = fused.shape[0]
    views = []
    for i in range(3):
        v = fused[:, i * H * D:(i + 1) * H * D].reshape(S_l, H, D)
        assert np.shares_memory(v, fused)
        views.append(v)
    return views


def unique_fused(P: int, S_l: int, H: int, D: int, pad: int = 0, base: int = 0):
    """Per-rank fused sources whose value columns hold distinct uint16 ids
    (distinct across ranks as well); padding columns hold SENTINEL."""
    hd3 = 3 * H * D
    n = P * S_l * hd3
    assert base + n <= 0x10000, "too many elements for unique 16-bit ids"
    ids = (np.arange(n, dtype=np.int64) + base).astype(np.uint16).reshape(P, S_l, hd3)
    out = []
    for r in range(P):
        f = np.full((S_l, hd3 + pad), SENTINEL, dtype=np.uint16)
        f[:, :hd3] = ids[r]
        out.append(f)
    return out


def unique_ids(n: int, base: int = 0) -> np.ndarray:
    assert base + n <= 0x10000
    return (np.arange(n, dtype=np.int64) + base).astype(np.uint16)


def random_u16(n: int, seed: int) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, 0x10000, size=n, dtype=np.uint16)


def padded_view(rows: int, heads: int, D: int, row_pad: int = 0, head_major: bool = False):
    """An output view [rows][heads][D] over a larger buffer pre-filled with
    SENTINEL.  Returns (view, backing buffer)."""
    if head_major:
        buf = np.full((heads, rows, D), SENTINEL, dtype=np.uint16)
        return buf.transpose(1, 0, 2), buf
    buf = np.full((rows, heads * D + row_pad), SENTINEL, dtype=np.uint16)
    return buf[:, :heads * D].reshape(rows, heads, D), buf
