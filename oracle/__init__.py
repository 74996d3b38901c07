"""ctypes access to the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The oracle performs the literal
materialised stack / permute / contiguous / cat chains that the Vflash
"Sol-Engine alignment" page ("What is enabled") says the direct relayout
replaces element for element.  It works on host numpy uint16 arrays holding
BF16 bit patterns.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


class Dims(ctypes.Structure):
    _fields_ = [("P", ctypes.c_int32), ("C", ctypes.c_int32), ("s_local", ctypes.c_int64),
                ("H", ctypes.c_int32), ("D", ctypes.c_int32)]


class View3(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_tok", ctypes.c_int64),
                ("stride_head", ctypes.c_int64)]


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        _lib = load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def library(path: str):
    """Temporarily routes this module's calls to another build of the oracle
    (the mutation tests use it to run the pins against planted mistakes)."""
    global _lib
    saved, _lib = _lib, load(path)
    try:
        yield
    finally:
        _lib = saved


def load(path: str) -> ctypes.CDLL:
    """Loads one build of the oracle and declares its signatures."""
    L = ctypes.CDLL(path)
    D, V, P = ctypes.POINTER(Dims), ctypes.POINTER(View3), ctypes.c_void_p
    i32, i64p = ctypes.c_int, ctypes.POINTER(ctypes.c_int64)
    L.oracle_qkv_pack.argtypes = [D, V, V, V, P, i32, i32, i64p]
    L.oracle_qkv_pack_permute.argtypes = [D, V, V, V, P]
    L.oracle_qkv_unpack.argtypes = [D, P, V, V, V, i32, i32, i64p]
    L.oracle_qkv_unpack_permute.argtypes = [D, P, V, V, V]
    L.oracle_attn_split.argtypes = [D, V, P, i32, i32, i64p]
    L.oracle_head_merge.argtypes = [D, P, V, i32, i32, i64p]
    L.oracle_exchange.argtypes = [D, i32, ctypes.POINTER(P), ctypes.POINTER(P)]
    L.oracle_set_threads.argtypes = [i32]
    L.oracle_set_threads.restype = None
    L.oracle_threads.argtypes = []
    L.oracle_qkv_pack_hc.argtypes = [D, V, V, V, P, i32, i32, i64p]
    L.oracle_qkv_unpack_hc.argtypes = [D, P, V, V, V, i32, i32, i64p]
    L.oracle_attn_split_hc.argtypes = [D, V, P, i32, i32, i64p]
    L.oracle_head_merge_hc.argtypes = [D, P, V, i32, i32, i64p]
    L.oracle_exchange_hc.argtypes = [D, i32, ctypes.POINTER(P), ctypes.POINTER(P)]
    for name in ("oracle_qkv_pack", "oracle_qkv_pack_permute", "oracle_qkv_unpack",
                 "oracle_qkv_unpack_permute", "oracle_attn_split", "oracle_head_merge",
                 "oracle_exchange", "oracle_threads", "oracle_qkv_pack_hc", "oracle_qkv_unpack_hc",
                 "oracle_attn_split_hc", "oracle_head_merge_hc", "oracle_exchange_hc"):
        getattr(L, name).restype = ctypes.c_int
    return L


def dims(P: int, C: int, s_local: int, H: int, D: int) -> Dims:
    return Dims(P, C, s_local, H, D)


def view(a: np.ndarray) -> View3:
    """A [tokens][heads][D] uint16 numpy view (unit stride on the last axis)."""
    if a.dtype != np.uint16 or a.ndim != 3 or a.strides[2] != 2:
        raise ValueError("oracle views are 3-D uint16 with a unit-stride last axis")
    return View3(a.ctypes.data, a.strides[0] // 2, a.strides[1] // 2)


def _ptr(a: np.ndarray) -> int:
    if a.dtype != np.uint16 or not a.flags.c_contiguous:
        raise ValueError("wire buffers are dense uint16")
    return a.ctypes.data


def _window(d: Dims, c_begin, c_end):
    return (0 if c_begin is None else c_begin), (d.C if c_end is None else c_end)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


def exchange_elems(d: Dims, which: int) -> int:
    """Elements in one rank's wire buffer: QKV (which=0) or attention return (1)."""
    return (3 if which == 0 else 1) * d.s_local * d.H * d.D


def _fn(name: str, chunk_heads: bool):
    """The token-chunked chain, or with chunk_heads the head-chunked one
    (chunks split each head group instead of the tokens)."""
    return getattr(lib(), name + ("_hc" if chunk_heads else ""))


def qkv_pack(d: Dims, q, k, v, packed, c_begin=None, c_end=None, chunk_heads=False) -> int:
    cb, ce = _window(d, c_begin, c_end)
    peak = ctypes.c_int64(0)
    _check(_fn("oracle_qkv_pack", chunk_heads)(ctypes.byref(d), view(q), view(k), view(v),
                                               _ptr(packed), cb, ce, ctypes.byref(peak)), "qkv_pack")
    return peak.value


def qkv_pack_permute(d: Dims, q, k, v, packed) -> None:
    _check(lib().oracle_qkv_pack_permute(ctypes.byref(d), view(q), view(k), view(v),
                                         _ptr(packed)), "qkv_pack_permute")


def qkv_unpack(d: Dims, recv, q, k, v, c_begin=None, c_end=None, chunk_heads=False) -> int:
    cb, ce = _window(d, c_begin, c_end)
    peak = ctypes.c_int64(0)
    _check(_fn("oracle_qkv_unpack", chunk_heads)(ctypes.byref(d), _ptr(recv), view(q), view(k),
                                                 view(v), cb, ce, ctypes.byref(peak)), "qkv_unpack")
    return peak.value


def qkv_unpack_permute(d: Dims, recv, q, k, v) -> None:
    _check(lib().oracle_qkv_unpack_permute(ctypes.byref(d), _ptr(recv), view(q), view(k),
                                           view(v)), "qkv_unpack_permute")


def attn_split(d: Dims, o, send, c_begin=None, c_end=None, chunk_heads=False) -> int:
    cb, ce = _window(d, c_begin, c_end)
    peak = ctypes.c_int64(0)
    _check(_fn("oracle_attn_split", chunk_heads)(ctypes.byref(d), view(o), _ptr(send), cb, ce,
                                                 ctypes.byref(peak)), "attn_split")
    return peak.value


def head_merge(d: Dims, recv, out, c_begin=None, c_end=None, chunk_heads=False) -> int:
    cb, ce = _window(d, c_begin, c_end)
    peak = ctypes.c_int64(0)
    _check(_fn("oracle_head_merge", chunk_heads)(ctypes.byref(d), _ptr(recv), view(out), cb, ce,
                                                 ctypes.byref(peak)), "head_merge")
    return peak.value


def exchange(d: Dims, which: int, sends, recvs, chunk_heads=False) -> None:
    arr = ctypes.c_void_p * d.P
    s = arr(*[_ptr(x) for x in sends])
    r = arr(*[_ptr(x) for x in recvs])
    _check(_fn("oracle_exchange", chunk_heads)(ctypes.byref(d), which, s, r), "exchange")


def set_threads(n: int) -> None:
    lib().oracle_set_threads(n)


def threads() -> int:
    return lib().oracle_threads()
