"""ctypes binding of liblinkmodel.so: the link-paced exchange of P virtual
ranks held in one GPU (harness/csrc/linkmodel.hip)."""
from __future__ import annotations

import ctypes
import os

from harness import build as _build

# xGMI on an eight-GPU MI355X node: one link per pair of GPUs, about 153 GB/s
# each way.
XGMI_LINK_GBS = 153.0


class Block(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p), ("bytes", ctypes.c_uint64),
                ("paced", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB_PATH):
            raise RuntimeError(f"{_build.LIB_PATH} is missing: build it with __graft_entry__.build()")
        import torch  # noqa: F401  (one HIP runtime: torch's)
        L = ctypes.CDLL(_build.LIB_PATH)
        L.lm_exchange.argtypes = [ctypes.POINTER(Block), ctypes.c_int32, ctypes.c_double, ctypes.c_void_p]
        L.lm_exchange.restype = ctypes.c_int
        L.lm_last_error.argtypes = []
        L.lm_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def exchange(pairs, link_gbs: float = XGMI_LINK_GBS) -> None:
    """Enqueues one paced exchange on the current stream.  pairs: (src, dst,
    paced) with src and dst same-size dense device tensors (views into wire
    buffers)."""
    import torch

    if not pairs:
        return
    blocks = (Block * len(pairs))()
    for i, (src, dst, paced) in enumerate(pairs):
        if not (src.is_cuda and dst.is_cuda and src.device == dst.device):
            raise ValueError("exchange blocks must be device tensors of one device")
        if src.numel() != dst.numel() or src.dtype != dst.dtype or not (src.is_contiguous() and dst.is_contiguous()):
            raise ValueError("exchange blocks must be dense and of equal size")
        blocks[i] = Block(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(), int(bool(paced)))
    stream = torch.cuda.current_stream().cuda_stream
    if lib().lm_exchange(blocks, len(pairs), float(link_gbs), stream) != 0:
        raise RuntimeError(f"lm_exchange: {lib().lm_last_error().decode()}")
