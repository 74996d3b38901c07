"""P virtual Ulysses ranks in one GPU: buffers, exchanges and schedules.

The stage order is the one the Vflash performance guide lists for the
sequence-head attention on the compute stream (section on profiling one
denoising request): QKV pack, inbound ready wait, QKV unpack, attention,
attention-result pack (split), outbound ready wait, final unpack (merge);
the collective runs on another stream and may overlap the pack or the
attention.  With the four-chunk overlap layout ("What is enabled" on the
Sol-Engine alignment page) each chunk is packed, exchanged and unpacked on
its own, so the exchange of chunk c overlaps the packing of chunk c + 1.
Attention itself is out of scope: the schedules pass one unpacked plane
through as the attention output (identity), which makes the whole path a
round trip that must return that plane of the input.
"""
from __future__ import annotations

import ctypes

import torch

import head_relayout_amd as vrl

# hipMemcpyKind asking the runtime for a device-to-device copy that uses no
# compute units (the SDMA engines) instead of a copy kernel.
_HIP_MEMCPY_D2D_NO_CU = 1024
_hip = None


def _hip_runtime() -> ctypes.CDLL:
    """The HIP runtime this process already uses (the one torch loaded, found
    by its mapped path), so that streams and pointers are that runtime's."""
    global _hip
    if _hip is None:
        name = "libamdhip64.so"
        with open("/proc/self/maps") as f:
            for line in f:
                path = line.split()[-1]
                if "/libamdhip64.so" in path:
                    name = path
                    break
        lib = ctypes.CDLL(name)
        lib.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                       ctypes.c_void_p]
        lib.hipMemcpyAsync.restype = ctypes.c_int
        _hip = lib
    return _hip


class Rank:
    """One virtual rank's device buffers (inputs are views of `fused`)."""

    def __init__(self, fused: torch.Tensor, P: int, C: int, H: int, D: int):
        S_l = fused.shape[0]
        self.fused = fused
        self.qkv = [fused[:, i * H * D:(i + 1) * H * D].unflatten(1, (H, D)) for i in range(3)]
        G, S = H // P, P * S_l
        bf = dict(dtype=torch.bfloat16, device=fused.device)
        n_qkv = vrl.exchange_elems(vrl.VRL_EXCHANGE_QKV, P, C, S_l, H, D)
        n_att = vrl.exchange_elems(vrl.VRL_EXCHANGE_ATTN, P, C, S_l, H, D)
        self.packed = torch.empty(n_qkv, **bf)
        self.recv = torch.empty(n_qkv, **bf)
        self.planes = [torch.empty(S, G, D, **bf) for _ in range(3)]
        self.send = torch.empty(n_att, **bf)
        self.back = torch.empty(n_att, **bf)
        self.merged = torch.empty(S_l, H, D, **bf)


class Layer:
    """Shapes and per-chunk wire offsets of P ranks' Ulysses exchange.

    engine: how the stand-in exchange copies blocks inside the one HBM --
    "kernel" (torch copies, run as copy kernels on the compute units),
    "sdma" (hipMemcpyAsync on the copy engines, no compute units) or "link"
    (one copy kernel per chunk that paces every block between two distinct
    ranks to link_gbs, each pair on a link of its own; harness/linkmodel.py).
    A real run moves the blocks over xGMI with RCCL instead."""

    def __init__(self, P: int, C: int, s_local: int, H: int, D: int, engine: str = "kernel",
                 link_gbs: float | None = None):
        if engine not in ("kernel", "sdma", "link"):
            raise ValueError(f"unknown exchange engine {engine!r}")
        if engine == "link" and P * P > 64:
            raise ValueError("the link-paced exchange takes at most 8 ranks")
        self.engine = engine
        if link_gbs is None:
            from harness.linkmodel import XGMI_LINK_GBS
            link_gbs = XGMI_LINK_GBS
        self.link_gbs = link_gbs
        self.P, self.C, self.s_local, self.H, self.D = P, C, s_local, H, D
        self.G = H // P
        self.off = [vrl.chunk_offset(c, P, C, s_local, H, D) for c in range(C + 1)]

    def block(self, x: int, c: int, per_token: int) -> slice:
        """Elements of wire block (peer x, chunk c): the peer's part holds the
        chunks of s_local tokens back to back, per_token elements each."""
        start = (x * self.s_local + self.off[c]) * per_token
        return slice(start, start + (self.off[c + 1] - self.off[c]) * per_token)

    def exchange(self, sends, recvs, qkv: bool, chunks=None) -> None:
        """recv_r[block (s, c)] = send_s[block (r, c)] for the given chunks."""
        per_token = (3 if qkv else 1) * self.G * self.D
        stream = torch.cuda.current_stream().cuda_stream
        for c in (range(self.C) if chunks is None else chunks):
            if self.engine == "link":
                from harness import linkmodel
                linkmodel.exchange([(sends[s][self.block(r, c, per_token)], recvs[r][self.block(s, c, per_token)],
                                     s != r) for s in range(self.P) for r in range(self.P)], self.link_gbs)
                continue
            for s in range(self.P):
                for r in range(self.P):
                    dst = recvs[r][self.block(s, c, per_token)]
                    src = sends[s][self.block(r, c, per_token)]
                    if self.engine == "kernel":
                        dst.copy_(src)
                        continue
                    rc = _hip_runtime().hipMemcpyAsync(dst.data_ptr(), src.data_ptr(), src.numel() * 2,
                                                      _HIP_MEMCPY_D2D_NO_CU, stream)
                    if rc != 0:
                        raise RuntimeError(f"hipMemcpyAsync failed with HIP error {rc}")


def run_exchanges(layer: Layer, ranks) -> None:
    """Only the layer's exchanges, chunk by chunk on the current stream (QKV,
    then the return path): the time the exchange alone takes."""
    for c in range(layer.C):
        layer.exchange([rk.packed for rk in ranks], [rk.recv for rk in ranks], True, [c])
    for c in range(layer.C):
        layer.exchange([rk.send for rk in ranks], [rk.back for rk in ranks], False, [c])


def run_serial(layer: Layer, ranks, plane: int = 0) -> None:
    """Every stage over all chunks at once, one stage after the other, on the
    current stream."""
    P, C = layer.P, layer.C
    for rk in ranks:
        vrl.qkv_pack(*rk.qkv, rk.packed, P, C)
    layer.exchange([rk.packed for rk in ranks], [rk.recv for rk in ranks], True)
    for rk in ranks:
        vrl.qkv_unpack(rk.recv, *rk.planes, P, C)
    for rk in ranks:
        vrl.attn_split(rk.planes[plane], rk.send, P, C)
    layer.exchange([rk.send for rk in ranks], [rk.back for rk in ranks], False)
    for rk in ranks:
        vrl.head_merge(rk.back, rk.merged, P, C)


def run_overlapped(layer: Layer, ranks, comm: torch.cuda.Stream, plane: int = 0,
                   waits: dict | None = None) -> None:
    """Per-chunk pack / exchange / unpack and split / exchange / merge, the
    exchanges on `comm`, ordered by events: a chunk's exchange waits for its
    pack (or split) on the compute stream; the compute stream waits for a
    chunk's exchange (inbound / outbound ready wait) before unpacking (or
    merging) it.  `waits`, if given, collects (before, after) event pairs
    around each ready wait on the compute stream."""
    P, C = layer.P, layer.C
    cs = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=waits is not None)  # noqa: E731

    def ready_wait(kind, e):
        if waits is not None:
            a, b = ev(), ev()
            a.record(cs)
            cs.wait_event(e)
            b.record(cs)
            waits.setdefault(kind, []).append((a, b))
        else:
            cs.wait_event(e)

    arrived = []
    for c in range(C):
        for rk in ranks:
            vrl.qkv_pack(*rk.qkv, rk.packed, P, C, c, c + 1)
        packed = ev()
        packed.record(cs)
        comm.wait_event(packed)
        with torch.cuda.stream(comm):
            layer.exchange([rk.packed for rk in ranks], [rk.recv for rk in ranks], True, [c])
        done = ev()
        done.record(comm)
        arrived.append(done)
    for c in range(C):
        ready_wait("inbound", arrived[c])
        for rk in ranks:
            vrl.qkv_unpack(rk.recv, *rk.planes, P, C, c, c + 1)
    returned = []
    for c in range(C):
        for rk in ranks:
            vrl.attn_split(rk.planes[plane], rk.send, P, C, c, c + 1)
        split = ev()
        split.record(cs)
        comm.wait_event(split)
        with torch.cuda.stream(comm):
            layer.exchange([rk.send for rk in ranks], [rk.back for rk in ranks], False, [c])
        done = ev()
        done.record(comm)
        returned.append(done)
    for c in range(C):
        ready_wait("outbound", returned[c])
        for rk in ranks:
            vrl.head_merge(rk.back, rk.merged, P, C, c, c + 1)
