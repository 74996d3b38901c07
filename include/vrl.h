/*
 * vrl: direct Ulysses sequence<->head relayout for MI355X (gfx950).
 *
 * C ABI of libvrl.so.  Four relayouts move BF16 tensors between a rank's
 * token-sharded, all-heads layout and the destination-major wire buffers of
 * a sequence-head (Ulysses) all-to-all, each in one strided read and one
 * write.  They replace the materialised stack/permute/contiguous (QKV pack)
 * and cat/permute/contiguous (returned-head merge) chains that the Vflash
 * "Sol-Engine alignment on SM86 and SM89" page describes under "What is
 * enabled", with identical output bits.  The order of the stages on the
 * compute stream (QKV pack, inbound wait, QKV unpack, attention, attention
 * result pack, outbound wait, final unpack) is the one listed in the
 * Vflash performance guide's section on profiling one denoising request.
 *
 * Notation.  P ranks, C chunks, S_l tokens per rank, S = P * S_l, H heads,
 * G = H / P heads per head group, D = head_dim.  Rank s holds global tokens
 * [s*S_l, (s+1)*S_l); dest rank d owns heads [d*G, (d+1)*G).  Chunks split a
 * rank's tokens by the tensor_split rule: with q = S_l / C and r = S_l % C,
 * chunk c has T(c) = q + (c < r) tokens and starts at off(c) = c*q + min(c, r).
 *
 * Wire layouts (dense, element offsets):
 *   QKV buffer    [P][C][3][T(c)][G][D]: block (d, c) starts at
 *                 (d*3*S_l + 3*off(c)) * G*D; plane q at +q*T(c)*G*D.
 *   return buffer [P][C][T(c)][G][D]:    block (d, c) starts at
 *                 (d*S_l + off(c)) * G*D.
 * In a send buffer the leading index is the destination rank, in a receive
 * buffer the source rank; the all-to-all moves block (r, c) of sender s to
 * block (s, c) of receiver r and is the caller's business (RCCL or a copy).
 *
 * Views.  A vrl_view describes a 3-D BF16 tensor [rows][heads][D] by its base
 * pointer and the element strides of its row (token) and head axes; the D
 * axis always has unit stride.  Any non-negative strides are accepted, so
 * fused projection outputs, padded rows and head-major storage are read or
 * written in place.
 *
 * Ownership.  The caller allocates every buffer on the current HIP device.
 * The library allocates no memory, keeps no pointer after a call returns and
 * holds no mutable global state besides a per-device architecture cache and
 * a per-thread error message, so calls are thread-safe.  Work is enqueued
 * asynchronously on `hip_stream` (a hipStream_t of the current device; NULL
 * is the null stream); buffers must stay alive until the stream has passed
 * the work.
 *
 * Windows.  Every relayout takes a chunk window [c_begin, c_end) with
 * 0 <= c_begin < c_end <= C; (0, C) is the whole tensor.  Only the window's
 * wire blocks, and the window's token rows (with chunk_heads, head columns)
 * of a view, are read and written; everything else, including padding
 * between a view's rows or heads, is left untouched.
 *
 * Errors.  All validation happens before anything is enqueued; on any error
 * nothing is launched and every output is unchanged.
 *   VRL_E_INVALID  bad dimensions (P, C, S_l, H, D < 1; H % P != 0; C > S_l
 *                  for token chunks; G % C != 0 for head chunks),
 *                  a bad window, a null pointer, a size beyond the supported
 *                  range, or a view that extends past the device allocation
 *                  holding its base pointer.  The allocation is what the HIP
 *                  runtime reports (hipMemGetAddressRange): a caching
 *                  allocator's segment can hold several tensors, and a view
 *                  that overruns its tensor but stays inside the segment is
 *                  accepted and written.  Strides that fit the caller's
 *                  tensors are the caller's responsibility.
 *   VRL_E_LAYOUT   an out-of-contract layout: a negative stride, an output
 *                  view whose elements overlap each other, overlapping output
 *                  views, an output that overlaps an input, or a pointer that
 *                  is not 2-byte aligned.  The caller keeps its reference
 *                  (materialising) path for such layouts; the library never
 *                  falls back silently.
 *   VRL_E_DEVICE   the current device is not gfx950, `hip_stream` or a
 *                  pointer belongs to another device, a pointer is not device
 *                  memory, or a HIP call failed.
 * No C++ exception crosses this interface.
 */
#ifndef VRL_H
#define VRL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VRL_OK = 0,
    VRL_E_INVALID = 1,
    VRL_E_LAYOUT = 2,
    VRL_E_DEVICE = 3
} vrl_status;

/* Problem size.  G = H / P must be a whole number.
 *
 * chunk_heads selects what the C chunks of the four-chunk overlap layout
 * split ("What is enabled" names the layout but not its axis):
 *   0  each rank's tokens (the layout above; C <= s_local);
 *   1  each destination's head group: chunk c holds heads [c*Gc, (c+1)*Gc)
 *      of the group, Gc = G / C (G % C == 0), for all S_l tokens.  The wire
 *      buffers are then [P][C][3][S_l][Gc][D] (QKV) and [P][C][S_l][Gc][D]
 *      (return): block (d, c) starts at (d*C + c) * 3*S_l*Gc*D, resp.
 *      (d*C + c) * S_l*Gc*D, and the four relayouts become
 *        packed[d][c][q][t][g][e]   = src_q[t][d*G + c*Gc + g][e]
 *        X_q[s*S_l + t][c*Gc + g][e] = recv[s][c][q][t][g][e]
 *        send[d][c][t][g][e]        = O[d*S_l + t][c*Gc + g][e]
 *        out[t][s*G + c*Gc + g][e]  = recv[s][c][t][g][e]
 * Buffer sizes (vrl_exchange_elems) are the same for both. */
typedef struct {
    int32_t P;           /* ranks (virtual ranks on one GPU)               */
    int32_t C;           /* chunks                                         */
    int64_t s_local;     /* tokens per rank, after padding                 */
    int32_t H;           /* attention heads                                */
    int32_t D;           /* head_dim                                       */
    int32_t chunk_heads; /* 0: chunks split tokens; 1: they split heads   */
} vrl_dims;

/* A [rows][heads][D] BF16 view; strides in elements, D stride is 1. */
typedef struct {
    void *ptr;
    int64_t stride_tok;
    int64_t stride_head;
} vrl_view;

enum { VRL_EXCHANGE_QKV = 0, VRL_EXCHANGE_ATTN = 1 };

/* Elements of one rank's wire buffer: 3*S_l*H*D for VRL_EXCHANGE_QKV,
 * S_l*H*D for VRL_EXCHANGE_ATTN.  Returns -1 for invalid arguments (the
 * dimension rules of VRL_E_INVALID below, or another `which`), with the
 * reason in vrl_last_error(). */
int64_t vrl_exchange_elems(int which, const vrl_dims *dims);

/* Start of chunk c along the chunked axis, for c in [0, C]: the first local
 * token off(c) (off(C) = S_l), or with chunk_heads the first head of the
 * chunk within a head group, c*Gc.  Returns -1 for invalid dimensions or c
 * outside [0, C], with the reason in vrl_last_error(). */
int64_t vrl_chunk_offset(const vrl_dims *dims, int32_t c);

/*
 * QKV destination pack (Vflash, "Sol-Engine alignment", section "What is
 * enabled": the direct kernel that reads the fused attn.qkv output's Q/K/V
 * views at their own strides and writes destination-major storage once).
 *   packed[d][c][q][t][g][e] = src_q[off(c) + t][d*G + g][e]
 * q, k, v: the rank's [S_l][H][D] inputs (read only; they may overlap each
 * other, e.g. column views of one fused projection row).
 * packed:  the rank's QKV send buffer, vrl_exchange_elems(VRL_EXCHANGE_QKV)
 *          elements.
 */
vrl_status vrl_qkv_pack(const vrl_dims *dims, const vrl_view *q, const vrl_view *k,
                        const vrl_view *v, void *packed, int32_t c_begin, int32_t c_end,
                        void *hip_stream);

/*
 * QKV unpack, the receive side (the "QKV unpack" compute-stream stage of the
 * performance guide's sequence-head profile), to BTHD with B = 1 and the
 * rank's G heads:
 *   X_q[s*S_l + off(c) + t][g][e] = recv[s][c][q][t][g][e]
 * recv:    the rank's QKV receive buffer (read only).
 * q, k, v: [S][G][D] outputs; they must not overlap each other or recv.
 */
vrl_status vrl_qkv_unpack(const vrl_dims *dims, const void *recv, const vrl_view *q,
                          const vrl_view *k, const vrl_view *v, int32_t c_begin, int32_t c_end,
                          void *hip_stream);

/*
 * Attention-result split (the "attention result split" row of the operation
 * table in "What is enabled"; the "attention result pack" stage of the
 * profile):
 *   send[d][c][t][g][e] = O[d*S_l + off(c) + t][g][e]
 * o:    the rank's [S][G][D] attention output (read only).
 * send: the rank's return send buffer, vrl_exchange_elems(VRL_EXCHANGE_ATTN)
 *       elements.
 */
vrl_status vrl_attn_split(const vrl_dims *dims, const vrl_view *o, void *send, int32_t c_begin,
                          int32_t c_end, void *hip_stream);

/*
 * Returned-head merge (the "returned-head merge" of "What is enabled"; the
 * "final unpack" stage of the profile):
 *   out[off(c) + t][s*G + g][e] = recv[s][c][t][g][e]
 * recv: the rank's return receive buffer (read only).
 * out:  the rank's [S_l][H][D] output; it must not overlap recv.
 */
vrl_status vrl_head_merge(const vrl_dims *dims, const void *recv, const vrl_view *out,
                          int32_t c_begin, int32_t c_end, void *hip_stream);

/* Static name of a status ("VRL_OK", ...). */
const char *vrl_status_string(vrl_status status);

/* Human-readable reason for the last non-OK status (or -1 from the two
 * sizing helpers) returned on the calling thread; empty after a call that
 * succeeded.  The string is owned by the library and valid until the
 * thread's next vrl call. */
const char *vrl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VRL_H */
