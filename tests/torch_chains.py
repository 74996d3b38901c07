"""The materialised chains written with PyTorch CPU library routines.

A second, library-based statement of the reference chains that the Vflash
"Sol-Engine alignment" page ("What is enabled") names: stack / permute /
contiguous for the QKV pack and cat / permute / contiguous for the returned
head merge.  Chunks come from torch.tensor_split itself, so this file holds
no chunk arithmetic of its own.  Tensors are int16 (BF16 bit patterns).
"""
from __future__ import annotations

import torch


def _chunk_lens(S_l: int, C: int):
    return [len(x) for x in torch.tensor_split(torch.arange(S_l), C)]


def pack(P, C, S_l, H, D, q, k, v):
    G = H // P
    X = torch.stack([q, k, v], 0)                       # [3][S_l][H][D]
    Xv = X.view(3, S_l, P, G, D)
    per_chunk = torch.tensor_split(Xv, C, dim=1)
    blocks = [per_chunk[c][:, :, d].contiguous().reshape(-1) for d in range(P) for c in range(C)]
    return torch.cat(blocks)


def unpack(P, C, S_l, H, D, recv):
    G = H // P
    lens = _chunk_lens(S_l, C)
    blocks = torch.split(recv, [3 * T * G * D for _ in range(P) for T in lens])
    shaped = [b.view(3, T, G, D) for b, T in zip(blocks, lens * P)]
    return [torch.cat([b[q] for b in shaped], 0) for q in range(3)]   # each [S][G][D]


def split(P, C, S_l, H, D, O):
    G = H // P
    Ov = O.reshape(P, S_l, G, D)
    parts = [t.contiguous().reshape(-1) for d in range(P) for t in torch.tensor_split(Ov[d], C, 0)]
    return torch.cat(parts)


def merge(P, C, S_l, H, D, recv):
    G = H // P
    Y = torch.stack([recv.view(P, S_l, G, D)[s] for s in range(P)], 0)   # [P][S_l][G][D]
    return Y.permute(1, 0, 2, 3).contiguous().view(S_l, H, D)


# ---- head-chunk reading: chunks split each head group (torch.tensor_split on heads)

def pack_hc(P, C, S_l, H, D, q, k, v):
    G = H // P
    Xv = torch.stack([q, k, v], 0).view(3, S_l, P, G, D)
    blocks = [blk.contiguous().reshape(-1) for d in range(P)
              for blk in torch.tensor_split(Xv[:, :, d], C, dim=2)]
    return torch.cat(blocks)


def unpack_hc(P, C, S_l, H, D, recv):
    Gc = H // P // C
    blocks = recv.view(P, C, 3, S_l, Gc, D)
    return [torch.cat([torch.cat([blocks[s, c, q] for c in range(C)], 1) for s in range(P)], 0)
            for q in range(3)]


def split_hc(P, C, S_l, H, D, O):
    G = H // P
    Ov = O.reshape(P, S_l, G, D)
    return torch.cat([blk.contiguous().reshape(-1) for d in range(P)
                      for blk in torch.tensor_split(Ov[d], C, dim=1)])


def merge_hc(P, C, S_l, H, D, recv):
    Gc = H // P // C
    Y = recv.view(P, C, S_l, Gc, D)
    return Y.permute(2, 0, 1, 3, 4).contiguous().view(S_l, H, D)
