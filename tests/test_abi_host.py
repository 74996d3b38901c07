"""Host-only checks of libvrl.so (no GPU, no kernel launch).

* the library loads and exports every function include/vrl.h declares;
* the host helpers (wire sizes, chunk offsets) agree with the tensor_split
  rule of torch and the index maps;
* every validation that precedes the device checks returns the documented
  status: dimensions, windows, NULLs, strides, alignment, overlaps and size
  limits.  Fake addresses are used: nothing is dereferenced or launched.
  Arguments that pass every host-side check reach the device check, which
  reports VRL_E_DEVICE on a machine without a GPU.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest
import torch

import head_relayout_amd as vrl
from head_relayout_amd import _lib
from tests import index_maps as im

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "vrl.h")
INVALID, LAYOUT, DEVICE = _lib.VRL_E_INVALID, _lib.VRL_E_LAYOUT, _lib.VRL_E_DEVICE

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-only: a visible GPU turns the device check into a pass")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vrl_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_function(vrl_lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (vrl_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(vrl_lib, name)


def test_status_strings(vrl_lib):
    assert [_lib.status_string(s) for s in range(4)] == [
        "VRL_OK", "VRL_E_INVALID", "VRL_E_LAYOUT", "VRL_E_DEVICE"]


def _d(P, C, S, H, D):
    return ctypes.byref(_lib.Dims(P, C, S, H, D))


@pytest.mark.parametrize("P,C,S,H,D", [(2, 4, 27707, 56, 128), (2, 4, 10, 4, 8), (4, 4, 7752, 32, 128),
                                       (3, 5, 5, 6, 8), (1, 1, 1, 1, 1), (8, 7, 1000, 64, 64)])
def test_host_helpers(vrl_lib, P, C, S, H, D):
    assert vrl_lib.vrl_exchange_elems(0, _d(P, C, S, H, D)) == 3 * S * H * D
    assert vrl_lib.vrl_exchange_elems(1, _d(P, C, S, H, D)) == S * H * D
    lens = [len(x) for x in torch.tensor_split(torch.arange(S), C)]
    starts = [sum(lens[:c]) for c in range(C + 1)]
    for c in range(C + 1):
        got = vrl_lib.vrl_chunk_offset(_d(P, C, S, H, D), c)
        assert got == starts[c]
        if c < C:
            assert got == im.off(S, C, c)
    assert vrl_lib.vrl_chunk_offset(_d(P, C, S, H, D), C + 1) == -1
    assert "outside" in _lib.last_error()
    assert vrl_lib.vrl_chunk_offset(_d(P, C, S, H, D), -1) == -1
    assert vrl_lib.vrl_exchange_elems(2, _d(P, C, S, H, D)) == -1
    assert "VRL_EXCHANGE_QKV" in _lib.last_error()
    assert vrl_lib.vrl_exchange_elems(0, _d(P, C, S, H, D)) > 0
    assert _lib.last_error() == ""


def test_sizing_errors_carry_the_reason():
    with pytest.raises(ValueError, match="not divisible"):
        vrl.exchange_elems(vrl.VRL_EXCHANGE_QKV, 3, 1, 8, 4, 8)
    with pytest.raises(ValueError, match="exceeds s_local"):
        vrl.chunk_offset(0, 2, 9, 8, 4, 8)
    with pytest.raises(ValueError, match="outside"):
        vrl.chunk_offset(5, 2, 4, 8, 4, 8)


BASE = 0x7F0000000000  # fake, 4 KiB aligned; never dereferenced


def V(ptr, st, sh):
    return ctypes.byref(_lib.View(ptr, st, sh))


def pack(L, dims, q, k, v, packed=BASE + (1 << 30), cb=0, ce=None):
    ce = dims[1] if ce is None else ce
    return L.vrl_qkv_pack(_d(*dims), q, k, v, packed, cb, ce, None)


def fused_qkv(dims, base=BASE, pad=0):
    P, C, S, H, D = dims
    row = 3 * H * D + pad
    return [V(base + 2 * i * H * D, row, D) for i in range(3)]


@pytest.mark.parametrize("dims", [(0, 1, 8, 4, 8), (2, 0, 8, 4, 8), (2, 1, 0, 4, 8), (2, 1, 8, 0, 8),
                                  (2, 1, 8, 4, 0), (3, 1, 8, 4, 8), (2, 9, 8, 4, 8)])
def test_invalid_dims(vrl_lib, dims):
    assert pack(vrl_lib, dims, *fused_qkv((2, 1, 8, 4, 8))) == INVALID
    assert _lib.last_error()


@pytest.mark.parametrize("cb,ce", [(-1, 2), (0, 5), (2, 2), (3, 1)])
def test_invalid_window(vrl_lib, cb, ce):
    dims = (2, 4, 16, 4, 8)
    assert pack(vrl_lib, dims, *fused_qkv(dims), cb=cb, ce=ce) == INVALID


def test_null_arguments(vrl_lib):
    dims = (2, 4, 16, 4, 8)
    q, k, v = fused_qkv(dims)
    assert vrl_lib.vrl_qkv_pack(None, q, k, v, BASE, 0, 4, None) == INVALID
    assert pack(vrl_lib, dims, q, None, v) == INVALID
    assert pack(vrl_lib, dims, q, k, V(0, 96, 8)) == INVALID
    assert pack(vrl_lib, dims, q, k, v, packed=None) == INVALID
    assert vrl_lib.vrl_head_merge(_d(*dims), None, V(BASE, 32, 8), 0, 4, None) == INVALID
    assert vrl_lib.vrl_attn_split(_d(*dims), None, BASE, 0, 4, None) == INVALID


def test_interleaved_fused_views_pass_host_checks(vrl_lib):
    # Q/K/V views of one fused row overlap in span but are legal inputs;
    # the call gets as far as the device check.
    dims = (2, 4, 16, 4, 8)
    assert pack(vrl_lib, dims, *fused_qkv(dims)) == DEVICE


def test_negative_stride_and_misalignment(vrl_lib):
    dims = (2, 4, 16, 4, 8)
    q, k, v = fused_qkv(dims)
    assert pack(vrl_lib, dims, V(BASE, -96, 8), k, v) == LAYOUT
    assert pack(vrl_lib, dims, q, k, V(BASE, 96, -8)) == LAYOUT
    assert pack(vrl_lib, dims, V(BASE + 1, 96, 8), k, v) == LAYOUT
    assert pack(vrl_lib, dims, q, k, v, packed=BASE + (1 << 30) + 1) == LAYOUT


def test_output_overlaps(vrl_lib):
    P, C, S_l, H, D = dims = (2, 4, 16, 4, 8)
    G, S = H // P, P * S_l
    L = vrl_lib
    recv = BASE + (1 << 30)
    # unpack outputs: interleaved in one [S][3][G][D] buffer is legal ...
    row = 3 * G * D
    ok = [V(BASE + 2 * i * G * D, row, D) for i in range(3)]
    assert L.vrl_qkv_unpack(_d(*dims), recv, *ok, 0, C, None) == DEVICE
    # ... the same view twice is not
    assert L.vrl_qkv_unpack(_d(*dims), recv, ok[0], ok[0], ok[2], 0, C, None) == LAYOUT
    # an output whose rows overlap each other
    assert L.vrl_qkv_unpack(_d(*dims), recv, V(BASE, G * D - 1, D), *ok[1:], 0, C, None) == LAYOUT
    # heads overlapping inside a row
    assert L.vrl_head_merge(_d(*dims), recv, V(BASE, H * D, D - 1), 0, C, None) == LAYOUT
    # a zero stride on an output
    assert L.vrl_head_merge(_d(*dims), recv, V(BASE, 0, D), 0, C, None) == LAYOUT
    # output overlapping the input wire buffer
    assert L.vrl_head_merge(_d(*dims), BASE + 64, V(BASE, H * D, D), 0, C, None) == LAYOUT
    # packed output overlapping an input view
    q, k, v = fused_qkv(dims)
    assert pack(L, dims, q, k, v, packed=BASE + 2 * 3 * H * D * 5) == LAYOUT
    # split output overlapping its input
    assert L.vrl_attn_split(_d(*dims), V(BASE, G * D, D), BASE + 2 * G * D * (S - 1), 0, C, None) \
        == LAYOUT
    # head-major output and a disjoint wire buffer are fine
    assert L.vrl_head_merge(_d(*dims), recv, V(BASE, D, S_l * D), 0, C, None) == DEVICE
    # broadcast (zero-stride) inputs are legal reads
    assert L.vrl_attn_split(_d(*dims), V(BASE, 0, 0), recv, 0, C, None) == DEVICE


def test_size_limits(vrl_lib):
    # one chunk of 2^25 tokens x 448 vectors exceeds the 2^31-vector tile index range
    dims = (2, 1, 1 << 25, 56, 128)
    q, k, v = fused_qkv(dims)
    assert pack(vrl_lib, dims, q, k, v, packed=BASE + (1 << 44)) == INVALID
    assert "too large" in _lib.last_error()
    # absurd totals are rejected by the dimension check
    assert pack(vrl_lib, (2, 1, 1 << 40, 56, 128), q, k, v) == INVALID


def _dh(P, C, S, H, D):
    return ctypes.byref(_lib.Dims(P, C, S, H, D, 1))


def test_head_chunk_validation(vrl_lib):
    L = vrl_lib
    # G = 4 divisible by C = 4: fine, even with more chunks than tokens
    dims = (2, 4, 3, 8, 8)
    q, k, v = fused_qkv(dims)
    assert L.vrl_qkv_pack(_dh(*dims), q, k, v, BASE + (1 << 30), 0, 4, None) == DEVICE
    # G = 4 not divisible by C = 3
    assert L.vrl_qkv_pack(_dh(2, 3, 9, 8, 8), q, k, v, BASE + (1 << 30), 0, 3, None) == INVALID
    assert "not divisible" in _lib.last_error()
    # chunk_heads other than 0 / 1
    bad = _lib.Dims(2, 2, 8, 8, 8, 2)
    assert L.vrl_qkv_pack(ctypes.byref(bad), q, k, v, BASE + (1 << 30), 0, 2, None) == INVALID
    # helpers
    assert [L.vrl_chunk_offset(_dh(2, 4, 27707, 56, 128), c) for c in range(5)] == [0, 7, 14, 21, 28]
    assert L.vrl_exchange_elems(0, _dh(2, 4, 27707, 56, 128)) == 3 * 27707 * 56 * 128
    assert L.vrl_exchange_elems(1, _dh(2, 3, 10, 8, 8)) == -1


def test_views_reaching_absurdly_far_are_rejected(vrl_lib):
    dims = (2, 4, 16, 4, 8)
    q, k, v = fused_qkv(dims)
    huge = V(BASE, 1 << 62, 8)
    assert pack(vrl_lib, dims, huge, k, v) == INVALID
    assert "2^48" in _lib.last_error()
    assert pack(vrl_lib, dims, q, k, V(BASE, 96, 1 << 60)) == INVALID


def test_error_reasons_are_per_thread(vrl_lib):
    """Calls from several threads at once: each thread's vrl_last_error names
    its own failing argument (the reason is thread-local; the library has no
    shared mutable state on these paths).  ctypes releases the GIL during a
    call, so the calls really overlap."""
    import threading

    errors = []

    def worker(t):
        # H = 4 * P + 1 is never divisible by P: every call fails with a reason naming H and P
        P = t + 2
        dims = (P, 1, 8, 4 * P + 1, 8)
        for _ in range(2000):
            if pack(vrl_lib, dims, *fused_qkv((2, 1, 8, 4, 8))) != INVALID:
                errors.append(f"thread {t}: unexpected status")
                return
            msg = _lib.last_error()
            if f"H={4 * P + 1}" not in msg or f"P={P}" not in msg:
                errors.append(f"thread {t}: reason {msg!r}")
                return

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
