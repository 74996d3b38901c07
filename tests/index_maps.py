"""Closed-form per-element index maps of the four relayouts (brute force).

An independent statement of what each relayout computes, written as a
direct address formula per output element rather than as a materialised
chain.  Used on tiny shapes to pin the oracle's chains.

Chunking follows the tensor_split rule: with q, r = divmod(S_l, C), chunk c
has T(c) = q + [c < r] tokens and starts at off(c) = c*q + min(c, r).

Wire layouts (destination-major, as the Vflash "Sol-Engine alignment" page's
"What is enabled" section describes, with the token-chunk reading):
  QKV:    block (d, c) starts at element (d*3*S_l + 3*off(c)) * G*D and is
          [3][T(c)][G][D];
  return: block (d, c) starts at element (d*S_l + off(c)) * G*D and is
          [T(c)][G][D].
With the head-chunk reading (chunks split each head group, Gc = G / C heads
per chunk) every block holds all S_l tokens:
  QKV:    block (d, c) starts at (d*C + c) * 3*S_l*Gc*D and is [3][S_l][Gc][D];
  return: block (d, c) starts at (d*C + c) * S_l*Gc*D and is [S_l][Gc][D].
"""
from __future__ import annotations

import numpy as np


def off(S_l: int, C: int, c: int) -> int:
    q, r = divmod(S_l, C)
    return c * q + min(c, r)


def tlen(S_l: int, C: int, c: int) -> int:
    q, r = divmod(S_l, C)
    return q + (1 if c < r else 0)


def pack(P, C, S_l, H, D, srcs, window=None, out=None):
    """packed[d][c][q][t][g][:] = src_q[off(c)+t][d*G+g][:]"""
    G = H // P
    cb, ce = window or (0, C)
    if out is None:
        out = np.zeros(3 * S_l * H * D, dtype=np.uint16)
    for d in range(P):
        for c in range(cb, ce):
            T, o = tlen(S_l, C, c), off(S_l, C, c)
            for q in range(3):
                for t in range(T):
                    for g in range(G):
                        at = ((d * 3 * S_l + 3 * o + q * T + t) * G + g) * D
                        out[at:at + D] = srcs[q][o + t, d * G + g, :]
    return out


def unpack(P, C, S_l, H, D, recv, outs, window=None):
    """X_q[s*S_l+off(c)+t][g][:] = recv[s][c][q][t][g][:]"""
    G = H // P
    cb, ce = window or (0, C)
    for s in range(P):
        for c in range(cb, ce):
            T, o = tlen(S_l, C, c), off(S_l, C, c)
            for q in range(3):
                for t in range(T):
                    for g in range(G):
                        at = ((s * 3 * S_l + 3 * o + q * T + t) * G + g) * D
                        outs[q][s * S_l + o + t, g, :] = recv[at:at + D]
    return outs


def split(P, C, S_l, H, D, o_view, window=None, out=None):
    """send[d][c][t][g][:] = O[d*S_l+off(c)+t][g][:]"""
    G = H // P
    cb, ce = window or (0, C)
    if out is None:
        out = np.zeros(S_l * H * D, dtype=np.uint16)
    for d in range(P):
        for c in range(cb, ce):
            T, o = tlen(S_l, C, c), off(S_l, C, c)
            for t in range(T):
                for g in range(G):
                    at = ((d * S_l + o + t) * G + g) * D
                    out[at:at + D] = o_view[d * S_l + o + t, g, :]
    return out


def merge(P, C, S_l, H, D, recv, out, window=None):
    """out[off(c)+t][s*G+g][:] = recv[s][c][t][g][:]"""
    G = H // P
    cb, ce = window or (0, C)
    for s in range(P):
        for c in range(cb, ce):
            T, o = tlen(S_l, C, c), off(S_l, C, c)
            for t in range(T):
                for g in range(G):
                    at = ((s * S_l + o + t) * G + g) * D
                    out[o + t, s * G + g, :] = recv[at:at + D]
    return out


def exchange(P, C, S_l, H, D, which, sends):
    """recv_r[s][c] = send_s[r][c]: block (r, c) of sender s -> block (s, c) of r."""
    G = H // P
    per_tok = (3 if which == 0 else 1) * G * D
    recvs = [np.zeros_like(sends[0]) for _ in range(P)]

    def start(x, c):
        return (x * S_l + off(S_l, C, c)) * per_tok

    for s in range(P):
        for r in range(P):
            for c in range(C):
                n = tlen(S_l, C, c) * per_tok
                recvs[r][start(s, c):start(s, c) + n] = sends[s][start(r, c):start(r, c) + n]
    return recvs


# ---- head-chunk reading ---------------------------------------------------------

def pack_hc(P, C, S_l, H, D, srcs, window=None, out=None):
    """packed[d][c][q][t][g][:] = src_q[t][d*G + c*Gc + g][:]"""
    G = H // P
    Gc = G // C
    cb, ce = window or (0, C)
    if out is None:
        out = np.zeros(3 * S_l * H * D, dtype=np.uint16)
    for d in range(P):
        for c in range(cb, ce):
            for q in range(3):
                for t in range(S_l):
                    for g in range(Gc):
                        at = ((((d * C + c) * 3 + q) * S_l + t) * Gc + g) * D
                        out[at:at + D] = srcs[q][t, d * G + c * Gc + g, :]
    return out


def unpack_hc(P, C, S_l, H, D, recv, outs, window=None):
    """X_q[s*S_l + t][c*Gc + g][:] = recv[s][c][q][t][g][:]"""
    G = H // P
    Gc = G // C
    cb, ce = window or (0, C)
    for s in range(P):
        for c in range(cb, ce):
            for q in range(3):
                for t in range(S_l):
                    for g in range(Gc):
                        at = ((((s * C + c) * 3 + q) * S_l + t) * Gc + g) * D
                        outs[q][s * S_l + t, c * Gc + g, :] = recv[at:at + D]
    return outs


def split_hc(P, C, S_l, H, D, o_view, window=None, out=None):
    """send[d][c][t][g][:] = O[d*S_l + t][c*Gc + g][:]"""
    G = H // P
    Gc = G // C
    cb, ce = window or (0, C)
    if out is None:
        out = np.zeros(S_l * H * D, dtype=np.uint16)
    for d in range(P):
        for c in range(cb, ce):
            for t in range(S_l):
                for g in range(Gc):
                    at = (((d * C + c) * S_l + t) * Gc + g) * D
                    out[at:at + D] = o_view[d * S_l + t, c * Gc + g, :]
    return out


def merge_hc(P, C, S_l, H, D, recv, out, window=None):
    """out[t][s*G + c*Gc + g][:] = recv[s][c][t][g][:]"""
    G = H // P
    Gc = G // C
    cb, ce = window or (0, C)
    for s in range(P):
        for c in range(cb, ce):
            for t in range(S_l):
                for g in range(Gc):
                    at = (((s * C + c) * S_l + t) * Gc + g) * D
                    out[t, s * G + c * Gc + g, :] = recv[at:at + D]
    return out


def exchange_hc(P, C, S_l, H, D, which, sends):
    """Block (r, c) of sender s -> block (s, c) of receiver r (equal blocks)."""
    Gc = H // P // C
    blk = (3 if which == 0 else 1) * S_l * Gc * D
    recvs = [np.zeros_like(sends[0]) for _ in range(P)]
    for s in range(P):
        for r in range(P):
            for c in range(C):
                recvs[r][(s * C + c) * blk:(s * C + c + 1) * blk] = \
                    sends[s][(r * C + c) * blk:(r * C + c + 1) * blk]
    return recvs
