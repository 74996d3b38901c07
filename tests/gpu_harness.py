"""Helpers for the GPU tests: host<->device BF16 bit copies, bit-exact
comparison on the device, guard bands and the simulated exchange."""
from __future__ import annotations

import sys

import numpy as np
import torch

SENTINEL = 0x7FC1
GUARD = 2048  # elements (4 KiB) of sentinel before and after a guarded buffer


def say(msg: str) -> None:
    """Progress line, flushed, so a GPU run's log names the case in flight."""
    print(msg, file=sys.stderr, flush=True)


def to_dev(a: np.ndarray, dev) -> torch.Tensor:
    """A bf16 device tensor holding the uint16 bit patterns of `a`."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(dev).view(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_bits_equal(got: torch.Tensor, want, what: str) -> None:
    """Element-by-element equality of BF16 bit patterns, on the device."""
    g = got.reshape(-1).view(torch.int16) if got.is_contiguous() else \
        got.contiguous().reshape(-1).view(torch.int16)
    if isinstance(want, np.ndarray):
        w = torch.from_numpy(np.ascontiguousarray(want).reshape(-1).view(np.int16)).to(got.device)
    else:
        w = want.contiguous().reshape(-1).view(torch.int16)
    assert g.numel() == w.numel(), f"{what}: {g.numel()} elements vs {w.numel()}"
    if not torch.equal(g, w):
        bad = (g != w).nonzero().reshape(-1)
        first = bad[:6].tolist()
        raise AssertionError(
            f"{what}: {bad.numel()} of {g.numel()} elements differ; first at {first}: "
            f"got {[hex(int(g[i]) & 0xFFFF) for i in first]} want {[hex(int(w[i]) & 0xFFFF) for i in first]}")


def guarded(numel: int, dev) -> tuple[torch.Tensor, torch.Tensor]:
    """A dense bf16 buffer of `numel` elements inside an allocation that has
    GUARD sentinel elements on each side.  Returns (inner, whole)."""
    whole = torch.full((numel + 2 * GUARD,), SENTINEL, dtype=torch.int16, device=dev)
    whole = whole.view(torch.bfloat16)
    return whole[GUARD:GUARD + numel], whole


def assert_guard_intact(whole: torch.Tensor, what: str) -> None:
    w = whole.view(torch.int16)
    assert bool((w[:GUARD] == SENTINEL).all()) and bool((w[-GUARD:] == SENTINEL).all()), \
        f"{what}: a guard band was written"


def sentinel_view(rows: int, heads: int, D: int, dev, row_pad: int = 0, head_major: bool = False):
    """A [rows][heads][D] bf16 view over a sentinel-filled buffer with padding
    (and guard bands around it).  Returns (view, whole buffer)."""
    if head_major:
        inner, whole = guarded(heads * rows * D, dev)
        return inner.view(heads, rows, D).transpose(0, 1), whole
    inner, whole = guarded(rows * (heads * D + row_pad), dev)
    return inner.view(rows, heads * D + row_pad)[:, :heads * D].unflatten(1, (heads, D)), whole


def sim_exchange(sends, recvs, P: int) -> None:
    """The all-to-all of P ranks' destination-major wire buffers, modelled in
    one HBM: the part of sender s addressed to r becomes the part of r's
    receive buffer that comes from s (each peer's part is 1/P of a buffer)."""
    for s in range(P):
        for r in range(P):
            recvs[r].view(P, -1)[s].copy_(sends[s].view(P, -1)[r])
