"""Seeded synthetic inputs shared by the oracle and the device path.

This module only draws values and lays them out as the workloads' source
tensors (fused QKV projection rows, standalone attention outputs).  It holds
no relayout arithmetic: no chunk offsets, head grouping or packing.

The workloads mirror the shapes of the Vflash "Sol-Engine alignment" page,
section "What is enabled": the representative 55,413-token Base16 shape
(two ranks, 56 heads of 128) and smaller / wider variants of it.  Values
are BF16 bit patterns held as numpy uint16.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdatagen.so")
_lib = None

# Written into the padding columns of a padded fused row; never a value the
# generators produce (a NaN with a payload), so it is easy to spot if copied.
PAD_SENTINEL = 0x7FC1


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name in ("dg_normal_bf16", "dg_uniform8_bf16"):
            f = getattr(L, name)
            f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64]
            f.restype = None
        L.dg_splitmix64.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64]
        L.dg_splitmix64.restype = None
        _lib = L
    return _lib


def fill(ptr: int, n: int, dist: str, seed: int, stream: int) -> None:
    """Fills n BF16 values at host address ptr from sequence (seed, stream)."""
    if dist == "normal":
        lib().dg_normal_bf16(ptr, n, seed, stream)
    elif dist == "uniform8":
        lib().dg_uniform8_bf16(ptr, n, seed, stream)
    else:
        raise ValueError(f"unknown distribution {dist!r}")


def values(n: int, dist: str = "normal", seed: int = 0, stream: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    if n:
        fill(out.ctypes.data, n, dist, seed, stream)
    return out


def splitmix64(n: int, state: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().dg_splitmix64(out.ctypes.data, n, state)
    return out


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: P ranks of a token-sharded sequence.

    total_tokens is padded up to P * s_local with zero-filled tail tokens;
    rank r holds global tokens [r * s_local, (r + 1) * s_local).  Each rank's
    source is a fused projection output of s_local rows, each row holding
    Q, K and V (H heads of D each, in that order) followed by row_pad padding
    columns filled with PAD_SENTINEL.
    """

    cid: int
    name: str
    P: int
    C: int
    s_local: int
    H: int
    D: int
    total_tokens: int
    seed: int
    dist: str = "normal"
    row_pad: int = 0

    @property
    def G(self) -> int:
        return self.H // self.P

    @property
    def S(self) -> int:
        return self.P * self.s_local

    @property
    def row_stride(self) -> int:
        return 3 * self.H * self.D + self.row_pad

    @property
    def n_pad_tokens(self) -> int:
        return self.S - self.total_tokens

    def dims(self) -> dict:
        return dict(P=self.P, C=self.C, s_local=self.s_local, H=self.H, D=self.D)


WORKLOADS = {
    1: Workload(1, "tiny round trip", P=2, C=1, s_local=64, H=4, D=16, total_tokens=128, seed=0),
    2: Workload(2, "mid-size", P=2, C=4, s_local=4096, H=32, D=128, total_tokens=8192, seed=2),
    3: Workload(3, "representative 55,413-token shape", P=2, C=4, s_local=27707, H=56, D=128,
                total_tokens=55413, seed=1),
    4: Workload(4, "strided fused source", P=2, C=4, s_local=27707, H=56, D=128,
                total_tokens=55413, seed=1, dist="uniform8", row_pad=64),
    5: Workload(5, "P=4 ragged", P=4, C=4, s_local=7752, H=32, D=128, total_tokens=31000, seed=5),
}


def fused_source(w: Workload, rank: int, out: np.ndarray | None = None) -> np.ndarray:
    """Rank `rank`'s fused source rows, uint16 [s_local][row_stride].

    Values come from stream `rank`; padding columns hold PAD_SENTINEL and the
    value columns of tail (padding) tokens are zero.  `out`, if given, is a
    C-contiguous uint16 array of that shape to fill (for example the numpy
    view of a pinned host tensor).
    """
    shape = (w.s_local, w.row_stride)
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    assert out.shape == shape and out.dtype == np.uint16 and out.flags.c_contiguous
    fill(out.ctypes.data, out.size, w.dist, w.seed, rank)
    hd3 = 3 * w.H * w.D
    if w.row_pad:
        out[:, hd3:] = PAD_SENTINEL
    first_pad = w.total_tokens - rank * w.s_local
    if first_pad < w.s_local:
        out[max(first_pad, 0):, :hd3] = 0
    return out


def attention_output(w: Workload, rank: int, out: np.ndarray | None = None) -> np.ndarray:
    """A standalone per-rank attention output, uint16 [S][G][D] (stream 100 + rank).

    Rows of global tokens beyond total_tokens are zero, as for the sources.
    """
    shape = (w.S, w.G, w.D)
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    assert out.shape == shape and out.dtype == np.uint16 and out.flags.c_contiguous
    fill(out.ctypes.data, out.size, w.dist, w.seed, 100 + rank)
    if w.total_tokens < w.S:
        out[w.total_tokens:] = 0
    return out
