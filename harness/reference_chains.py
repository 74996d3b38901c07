"""The reference materialisation chains, run on the GPU with torch-ROCm.

The Vflash "Sol-Engine alignment on SM86 and SM89" page (section "What is
enabled", the operation table and the allocation-screen paragraph after it)
compares each direct relayout with the chain it replaces: the QKV pack as a
stack, permute and contiguous, the returned-head merge as a cat, permute and
contiguous, the split as a per-chunk materialisation.  These functions are
those chains written with torch operations on device tensors.  They are a
comparison arm for the benchmark and its tests only; the library never calls
them and never falls back to them.

Layouts are the library's (token chunks): the QKV wire buffer is
[dest][chunk][q/k/v][token][head_group][D], the return wire buffer
[peer][chunk][token][head_group][D]; chunk sizes follow torch.tensor_split.
"""
from __future__ import annotations


def ref_pack(torch, q, k, v, P, C):
    """stack, then each (dest, chunk) block copied into its slot of a new
    buffer: two materialisations (the stacked tensor and the packed one)."""
    S_l, H, D = q.shape
    X = torch.stack([q, k, v], 0)
    Xv = X.view(3, S_l, P, H // P, D)
    out = torch.empty(3 * S_l * H * D, dtype=q.dtype, device=q.device)
    at = 0
    for d in range(P):
        for blk in torch.tensor_split(Xv[:, :, d], C, dim=1):
            n = blk.numel()
            out[at:at + n].view(blk.shape).copy_(blk)
            at += n
    return out


def ref_unpack(torch, recv, P, C, S_l, G, D):
    """per plane, cat of the received blocks: one materialisation per plane."""
    lens = [len(x) for x in torch.tensor_split(torch.arange(S_l), C)]
    blocks = torch.split(recv, [3 * T * G * D for _ in range(P) for T in lens])
    shaped = [b.view(3, T, G, D) for b, T in zip(blocks, lens * P)]
    return [torch.cat([b[q] for b in shaped], 0) for q in range(3)]


def ref_split(torch, o, P, C, c_begin=0, c_end=None):
    """cat of each (dest, chunk) token slice of O for the chunks in
    [c_begin, c_end): one materialisation, the window's blocks back to back
    (destination-major)."""
    S, G, D = o.shape
    Ov = o.view(P, S // P, G, D)
    parts = []
    for d in range(P):
        chunks = torch.tensor_split(Ov[d], C, 0)
        parts += [x.reshape(-1) for x in chunks[c_begin:c_end]]
    return torch.cat(parts)


def ref_merge(torch, recv, P, S_l, G, D):
    """stack of the per-source head groups, then permute + contiguous: two
    materialisations."""
    Y = torch.stack([recv.view(P, S_l, G, D)[s] for s in range(P)], 0)
    return Y.permute(1, 0, 2, 3).contiguous().view(S_l, P * G, D)


def peak_bytes(torch, fn) -> int:
    """Incremental peak of device memory that the caching allocator hands
    out while fn() runs and its result is alive (the result included)."""
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    out = fn()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    del out
    return peak
