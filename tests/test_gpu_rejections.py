"""Rejected calls on the GPU: every validation that needs the device
(allocation extents, host pointers) returns its status and writes nothing.

The first test checks, without launching anything, that the HIP runtime
reports the extent of a device allocation the way the library's extent check
relies on; the rejection tests run only after it.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import head_relayout_amd as vrl
from head_relayout_amd import _lib
from tests.gpu_harness import assert_guard_intact, guarded, say, to_dev
from tests.pipeline import dev_qkv

pytestmark = pytest.mark.gpu


def test_allocation_range_query(gpu):
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipMemGetAddressRange.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    for n in (1000, 5_000_000, 50_000_000):
        t = torch.empty(n, dtype=torch.bfloat16, device=gpu)
        base, size = ctypes.c_void_p(), ctypes.c_size_t()
        assert hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size),
                                         t.data_ptr() + 2 * (n // 2)) == 0
        # the range is the allocation (a caching allocator's segment may be
        # larger than the tensor) and contains the whole tensor
        assert base.value <= t.data_ptr()
        assert base.value + size.value >= t.data_ptr() + 2 * n
    say("allocation range query ok")


def _d(P, C, S, H, D):
    return ctypes.byref(_lib.Dims(P, C, S, H, D))


def _v(t_or_ptr, st, sh):
    ptr = t_or_ptr if isinstance(t_or_ptr, int) else t_or_ptr.data_ptr()
    return ctypes.byref(_lib.View(ptr, st, sh))


def _hip():
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipFree.argtypes = [ctypes.c_void_p]
    hip.hipMemGetAddressRange.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    return hip


def test_view_past_allocation_rejected(gpu):
    """An input view whose last row lies past the end of its allocation is
    rejected (VRL_E_INVALID) before anything is launched.  The output sits at
    the start of the same allocation, so no overlap check can fire first."""
    hip = _hip()
    torch.zeros(1, device=gpu)  # make the device current
    region = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(region), 1 << 20) == 0
    try:
        base, size = ctypes.c_void_p(), ctypes.c_size_t()
        assert hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), region.value) == 0
        assert base.value == region.value and size.value == 1 << 20
        P, C, S_l, H, D = 2, 2, 16, 4, 8
        G, S = H // P, P * S_l
        send = base.value
        o_bytes = 2 * S * G * D
        o_ptr = base.value + size.value - o_bytes + 2 * G * D   # one row past the end
        st = _lib.lib().vrl_attn_split(_d(P, C, S_l, H, D), _v(o_ptr, G * D, D), send, 0, C, None)
        assert st == _lib.VRL_E_INVALID, _lib.last_error()
        assert "past its allocation" in _lib.last_error()
        # the same call one row earlier is in bounds and runs
        st = _lib.lib().vrl_attn_split(_d(P, C, S_l, H, D), _v(o_ptr - 2 * G * D, G * D, D), send,
                                       0, C, None)
        assert st == _lib.VRL_OK, _lib.last_error()
        torch.cuda.synchronize()
    finally:
        torch.cuda.synchronize()
        hip.hipFree(region.value)


def test_rejected_calls_write_nothing(gpu):
    L = _lib.lib()
    P, C, S_l, H, D = 2, 4, 16, 4, 8
    G = H // P
    src = to_dev(np.arange(S_l * 3 * H * D, dtype=np.uint16), gpu)
    row = 3 * H * D
    q, k, v = (_v(src.data_ptr() + 2 * i * H * D, row, D) for i in range(3))
    n = 3 * S_l * H * D
    packed, whole = guarded(n, gpu)
    before = whole.clone()

    def untouched(what):
        torch.cuda.synchronize()
        assert torch.equal(whole.view(torch.int16), before.view(torch.int16)), what

    # host memory passed as a device pointer
    host = np.zeros(n, dtype=np.uint16)
    assert L.vrl_qkv_pack(_d(P, C, S_l, H, D), _v(host.ctypes.data, row, D), k, v, packed.data_ptr(),
                          0, C, None) == _lib.VRL_E_DEVICE
    untouched("host pointer")
    # output overlapping an input
    assert L.vrl_qkv_pack(_d(P, C, S_l, H, D), q, k, v, src.data_ptr() + 64, 0, C, None) \
        == _lib.VRL_E_LAYOUT
    # bad window
    assert L.vrl_qkv_pack(_d(P, C, S_l, H, D), q, k, v, packed.data_ptr(), 2, 2, None) \
        == _lib.VRL_E_INVALID
    untouched("bad window")
    # the binding raises, naming the status
    with pytest.raises(vrl.VrlError, match="VRL_E_INVALID"):
        vrl.qkv_pack(*dev_qkv(src.view(S_l, row), H, D), packed, P, C, 3, 2)
    untouched("binding")
    # a valid call on the same buffers then succeeds
    vrl.qkv_pack(*dev_qkv(src.view(S_l, row), H, D), packed, P, C)
    torch.cuda.synchronize()
    assert_guard_intact(whole, "valid call after rejections")
    say("rejections ok")


def test_extent_check_is_per_allocation(gpu):
    """The extent check compares each view with the device allocation that
    holds it (as hipMemGetAddressRange reports it; under torch's caching
    allocator that is a segment, which may hold several tensors), not with
    the tensor the caller means.  An output view that runs past its tensor
    into a neighbouring tensor of the same allocation is therefore accepted
    and writes there; one that runs past the allocation's end is rejected
    with VRL_E_INVALID and writes nothing."""
    from tests.gpu_harness import SENTINEL

    L = _lib.lib()
    P, C, S_l, H, D = 2, 2, 8, 4, 8
    n = S_l * H * D
    recv = to_dev(np.arange(1, n + 1, dtype=np.uint16), gpu)

    # inside one allocation: x and its neighbour are views of one tensor
    arena = torch.full((3 * n,), SENTINEL, dtype=torch.int16, device=gpu)
    x = arena[n:2 * n]
    st = H * D + 1          # rows one element too far apart: the last row ends past x
    assert L.vrl_head_merge(_d(P, C, S_l, H, D), recv.data_ptr(), _v(x.data_ptr(), st, D), 0, C, None) \
        == _lib.VRL_OK, _lib.last_error()
    torch.cuda.synchronize()
    end = (S_l - 1) * st + H * D            # elements of the view's span, from x's start
    assert end > n
    assert bool((arena[2 * n:n + end] != SENTINEL).any()), "the over-reach did not reach the neighbour"
    assert bool((arena[:n] == SENTINEL).all()) and bool((arena[n + end:] == SENTINEL).all())

    # past the allocation: a hipMalloc'd region filled with 0xAB bytes
    hip = _hip()
    hip.hipMemset.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t]
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipDeviceSynchronize.argtypes = []
    region = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(region), 1 << 20) == 0
    try:
        base, size = ctypes.c_void_p(), ctypes.c_size_t()
        assert hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), region.value) == 0
        # the runtime's range is exactly this allocation (else the views below
        # would be placed relative to memory this test does not own)
        assert base.value == region.value and size.value == 1 << 20
        assert hip.hipMemset(region.value, 0xAB, size.value) == 0
        assert hip.hipDeviceSynchronize() == 0
        out = base.value + size.value - 2 * n + 2 * H * D        # the last row one row past the end
        assert L.vrl_head_merge(_d(P, C, S_l, H, D), recv.data_ptr(), _v(out, H * D, D), 0, C, None) \
            == _lib.VRL_E_INVALID
        assert "past its allocation" in _lib.last_error()
        assert hip.hipDeviceSynchronize() == 0
        host = np.empty(size.value, np.uint8)
        assert hip.hipMemcpy(host.ctypes.data, base.value, size.value, 2) == 0   # device to host
        assert bool((host == 0xAB).all()), "a rejected call wrote into the allocation"
        # one row earlier the view fits and the call runs
        assert L.vrl_head_merge(_d(P, C, S_l, H, D), recv.data_ptr(), _v(out - 2 * H * D, H * D, D), 0, C,
                                None) == _lib.VRL_OK, _lib.last_error()
        assert hip.hipDeviceSynchronize() == 0
    finally:
        torch.cuda.synchronize()
        hip.hipFree(region.value)
    say("extent check per allocation ok")
