"""Direct Ulysses sequence<->head relayout for MI355X (gfx950).

A thin binding over libvrl.so (include/vrl.h): it turns torch tensors into
pointers, strides and a HIP stream handle and calls the library; every
element is moved by the library's HIP kernels.  There is no other code path:
if the library is missing, or a call fails validation, an exception is
raised.

The four calls follow the relayouts of the Vflash "Sol-Engine alignment on
SM86 and SM89" page ("What is enabled") and the compute-stream stage list of
its performance guide (QKV pack, QKV unpack, attention-result split,
returned-head merge).  Tensors are torch.bfloat16 on the current HIP device
with a unit-stride last axis; views may have any non-negative strides
otherwise.  Wire buffers are dense, with exchange_elems(...) elements.
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import (VRL_E_DEVICE, VRL_E_INVALID, VRL_E_LAYOUT, VRL_EXCHANGE_ATTN,
                   VRL_EXCHANGE_QKV, VRL_OK, VrlError)

__all__ = ["qkv_pack", "qkv_unpack", "attn_split", "head_merge", "exchange_elems",
           "chunk_offset", "VrlError", "VRL_OK", "VRL_E_INVALID", "VRL_E_LAYOUT",
           "VRL_E_DEVICE", "VRL_EXCHANGE_QKV", "VRL_EXCHANGE_ATTN"]


def _torch():
    import torch
    return torch


def _dims(P, C, s_local, H, D, chunk_heads=False) -> _lib.Dims:
    return _lib.Dims(int(P), int(C), int(s_local), int(H), int(D), int(bool(chunk_heads)))


def _view(t, name: str) -> _lib.View:
    torch = _torch()
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be torch.bfloat16, got {t.dtype}")
    if t.device.type != "cuda":
        raise TypeError(f"{name} must be a HIP device tensor")
    if t.dim() == 4 and t.shape[0] == 1:      # BTHD with B = 1
        t = t[0]
    if t.dim() != 3:
        raise ValueError(f"{name} must be [tokens][heads][D], got shape {tuple(t.shape)}")
    if t.shape[2] > 1 and t.stride(2) != 1:
        raise ValueError(f"{name} must have a unit-stride last axis")
    return _lib.View(t.data_ptr(), t.stride(0), t.stride(1))


def _wire(t, elems: int, name: str) -> int:
    torch = _torch()
    if t.dtype != torch.bfloat16 or t.device.type != "cuda":
        raise TypeError(f"{name} must be a torch.bfloat16 HIP device tensor")
    if not t.is_contiguous() or t.numel() != elems:
        raise ValueError(f"{name} must be dense with {elems} elements")
    return t.data_ptr()


def _stream(stream, device) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _window(C, c_begin, c_end):
    return int(c_begin), int(C if c_end is None else c_end)


def exchange_elems(which: int, P: int, C: int, s_local: int, H: int, D: int,
                   chunk_heads: bool = False) -> int:
    """Elements of one rank's wire buffer (which: VRL_EXCHANGE_QKV or _ATTN)."""
    n = _lib.lib().vrl_exchange_elems(which, ctypes.byref(_dims(P, C, s_local, H, D, chunk_heads)))
    if n < 0:
        raise ValueError(f"invalid dimensions: {_lib.last_error()}")
    return n


def chunk_offset(c: int, P: int, C: int, s_local: int, H: int, D: int,
                 chunk_heads: bool = False) -> int:
    """Start of chunk c along the chunked axis: its first local token (c = C
    gives s_local), or with chunk_heads its first head within a head group."""
    n = _lib.lib().vrl_chunk_offset(ctypes.byref(_dims(P, C, s_local, H, D, chunk_heads)), int(c))
    if n < 0:
        raise ValueError(f"invalid arguments: {_lib.last_error()}")
    return n


def qkv_pack(q, k, v, packed, P: int, C: int, c_begin: int = 0, c_end: int | None = None,
             stream=None, chunk_heads: bool = False) -> None:
    """packed[d][c][q][t][g][:] = src_q[off(c)+t][d*G+g][:]; q, k, v are [S_l][H][D].
    With chunk_heads the chunks split head groups (see include/vrl.h)."""
    S_l, H, D = q.shape[-3], q.shape[-2], q.shape[-1]
    d = _dims(P, C, S_l, H, D, chunk_heads)
    vq, vk, vv = _view(q, "q"), _view(k, "k"), _view(v, "v")
    for t, n in ((k, "k"), (v, "v")):
        if tuple(t.shape[-3:]) != (S_l, H, D):
            raise ValueError(f"{n} must have the shape of q")
    cb, ce = _window(C, c_begin, c_end)
    ptr = _wire(packed, exchange_elems(VRL_EXCHANGE_QKV, P, C, S_l, H, D, chunk_heads), "packed")
    _lib.check(_lib.lib().vrl_qkv_pack(ctypes.byref(d), ctypes.byref(vq), ctypes.byref(vk),
                                       ctypes.byref(vv), ptr, cb, ce, _stream(stream, q.device)),
               "vrl_qkv_pack")


def qkv_unpack(recv, q, k, v, P: int, C: int, c_begin: int = 0, c_end: int | None = None,
               stream=None, chunk_heads: bool = False) -> None:
    """X_q[s*S_l+off(c)+t][g][:] = recv[s][c][q][t][g][:]; q, k, v are [S][G][D] (or [1][S][G][D])."""
    S, G, D = q.shape[-3], q.shape[-2], q.shape[-1]
    if S % P:
        raise ValueError("the token count of q must be a multiple of P")
    d = _dims(P, C, S // P, G * P, D, chunk_heads)
    vq, vk, vv = _view(q, "q"), _view(k, "k"), _view(v, "v")
    for t, n in ((k, "k"), (v, "v")):
        if tuple(t.shape[-3:]) != (S, G, D):
            raise ValueError(f"{n} must have the shape of q")
    cb, ce = _window(C, c_begin, c_end)
    ptr = _wire(recv, exchange_elems(VRL_EXCHANGE_QKV, P, C, S // P, G * P, D, chunk_heads), "recv")
    _lib.check(_lib.lib().vrl_qkv_unpack(ctypes.byref(d), ptr, ctypes.byref(vq), ctypes.byref(vk),
                                         ctypes.byref(vv), cb, ce, _stream(stream, q.device)),
               "vrl_qkv_unpack")


def attn_split(o, send, P: int, C: int, c_begin: int = 0, c_end: int | None = None,
               stream=None, chunk_heads: bool = False) -> None:
    """send[d][c][t][g][:] = O[d*S_l+off(c)+t][g][:]; o is [S][G][D] (or [1][S][G][D])."""
    S, G, D = o.shape[-3], o.shape[-2], o.shape[-1]
    if S % P:
        raise ValueError("the token count of o must be a multiple of P")
    d = _dims(P, C, S // P, G * P, D, chunk_heads)
    vo = _view(o, "o")
    cb, ce = _window(C, c_begin, c_end)
    ptr = _wire(send, exchange_elems(VRL_EXCHANGE_ATTN, P, C, S // P, G * P, D, chunk_heads), "send")
    _lib.check(_lib.lib().vrl_attn_split(ctypes.byref(d), ctypes.byref(vo), ptr, cb, ce,
                                         _stream(stream, o.device)), "vrl_attn_split")


def head_merge(recv, out, P: int, C: int, c_begin: int = 0, c_end: int | None = None,
               stream=None, chunk_heads: bool = False) -> None:
    """out[off(c)+t][s*G+g][:] = recv[s][c][t][g][:]; out is [S_l][H][D]."""
    S_l, H, D = out.shape[-3], out.shape[-2], out.shape[-1]
    d = _dims(P, C, S_l, H, D, chunk_heads)
    vo = _view(out, "out")
    cb, ce = _window(C, c_begin, c_end)
    ptr = _wire(recv, exchange_elems(VRL_EXCHANGE_ATTN, P, C, S_l, H, D, chunk_heads), "recv")
    _lib.check(_lib.lib().vrl_head_merge(ctypes.byref(d), ptr, ctypes.byref(vo), cb, ce,
                                         _stream(stream, out.device)), "vrl_head_merge")
