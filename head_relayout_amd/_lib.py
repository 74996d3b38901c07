"""ctypes declarations of libvrl.so (the C ABI in include/vrl.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvrl.so")

VRL_OK, VRL_E_INVALID, VRL_E_LAYOUT, VRL_E_DEVICE = 0, 1, 2, 3
VRL_EXCHANGE_QKV, VRL_EXCHANGE_ATTN = 0, 1

# Every function include/vrl.h declares.
EXPORTS = ("vrl_exchange_elems", "vrl_chunk_offset", "vrl_qkv_pack", "vrl_qkv_unpack",
           "vrl_attn_split", "vrl_head_merge", "vrl_status_string", "vrl_last_error")


class Dims(ctypes.Structure):
    _fields_ = [("P", ctypes.c_int32), ("C", ctypes.c_int32), ("s_local", ctypes.c_int64),
                ("H", ctypes.c_int32), ("D", ctypes.c_int32), ("chunk_heads", ctypes.c_int32)]


class View(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_tok", ctypes.c_int64),
                ("stride_head", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libvrl.so; raises if it has not been built (there is no other path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        # torch ships a HIP runtime with the same soname as the system one;
        # loading torch first makes the process use exactly one runtime, the
        # one that owns torch's allocations and streams.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        D, V, P, i32 = ctypes.POINTER(Dims), ctypes.POINTER(View), ctypes.c_void_p, ctypes.c_int32
        L.vrl_exchange_elems.argtypes = [ctypes.c_int, D]
        L.vrl_exchange_elems.restype = ctypes.c_int64
        L.vrl_chunk_offset.argtypes = [D, i32]
        L.vrl_chunk_offset.restype = ctypes.c_int64
        L.vrl_qkv_pack.argtypes = [D, V, V, V, P, i32, i32, P]
        L.vrl_qkv_unpack.argtypes = [D, P, V, V, V, i32, i32, P]
        L.vrl_attn_split.argtypes = [D, V, P, i32, i32, P]
        L.vrl_head_merge.argtypes = [D, P, V, i32, i32, P]
        for f in (L.vrl_qkv_pack, L.vrl_qkv_unpack, L.vrl_attn_split, L.vrl_head_merge):
            f.restype = ctypes.c_int
        L.vrl_status_string.argtypes = [ctypes.c_int]
        L.vrl_status_string.restype = ctypes.c_char_p
        L.vrl_last_error.argtypes = []
        L.vrl_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().vrl_status_string(status).decode()


def last_error() -> str:
    return lib().vrl_last_error().decode()


class VrlError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}: {last_error()}")


def check(status: int, what: str) -> None:
    if status != VRL_OK:
        raise VrlError(status, what)
