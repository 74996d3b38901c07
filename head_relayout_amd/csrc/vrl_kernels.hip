// gfx950 kernels of the direct sequence<->head relayout.
//
// All four relayouts (Vflash, "Sol-Engine alignment on SM86 and SM89",
// section "What is enabled": QKV destination pack, attention-result split,
// returned-head merge; plus the receive-side QKV unpack named in the
// performance guide's sequence-head profile) are one batched copy between a
// dense wire block [T(c)][G][D] and a strided region of a caller's view:
//
//   wire row (token t of the block)  <->  view row: G heads of D elements at
//                                         token tok0 + t, heads head0 ..
//
// Pack and merge touch the [S_l][H][D] side (dest/source rank selects the
// head group), unpack and split the [S][G][D] side (rank selects the token
// range).  Pack and split gather view -> wire, unpack and merge scatter
// wire -> view.  Only integer moves: BF16 bit patterns travel in 2..16-byte
// unsigned vectors and never through float registers, so -0, subnormals and
// NaN payloads are preserved.
//
// Mapping to CDNA4.  One workgroup (256 lanes, four wave64s) moves one tile
// of kTileVecs consecutive vectors of one wire block; the grid is flattened
// over (rank, chunk, plane, token tile).  Lanes take consecutive 16-byte
// vectors, so a wave64 moves 1 KiB per instruction: four 128-element head
// rows, contiguous on the wire side and, for head-contiguous views, on the
// view side as well.  Each lane first issues all of its kUnroll loads and
// only then its stores, which keeps 32 KiB per workgroup in flight.  The
// dense wire offset of vector f is f itself; the view offset needs f's row
// and column, obtained with a precomputed multiply-shift division.  Address
// arithmetic is 64-bit wherever a product can pass 2^31 elements.
#include "vrl_internal.h"

namespace vrl {
namespace {

template <int VB>
struct Vec;
template <>
struct Vec<16> {
    typedef uint32_t type __attribute__((ext_vector_type(4)));
};
template <>
struct Vec<8> {
    typedef uint32_t type __attribute__((ext_vector_type(2)));
};
template <>
struct Vec<4> {
    typedef uint32_t type;
};
template <>
struct Vec<2> {
    typedef uint16_t type;
};

#ifndef VRL_RANK_INNER
#define VRL_RANK_INNER 1
#endif
#ifndef VRL_PLANE_INNER
#define VRL_PLANE_INNER 0
#endif

// Streaming cache policy: every byte is touched exactly once.
#ifndef VRL_LOAD_NT
#define VRL_LOAD_NT 1
#endif
#ifndef VRL_STORE_NT
#define VRL_STORE_NT 1
#endif

template <typename V>
__device__ __forceinline__ V load_vec(const V *p)
{
#if VRL_LOAD_NT
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

template <typename V>
__device__ __forceinline__ void store_vec(V *p, V v)
{
#if VRL_STORE_NT
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// n / d for n < 2^31, with magic = ceil(2^shift / d), shift = 31 + ceil(log2 d):
// the rounding error n * (magic * d - 2^shift) stays below 2^shift.
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint64_t magic, uint32_t shift)
{
    return uint32_t((uint64_t(n) * magic) >> shift);
}

template <Op OP>
struct Traits;
template <>
struct Traits<Op::Pack> {
    static constexpr bool gather = true, hside = true, planes3 = true;
};
template <>
struct Traits<Op::Unpack> {
    static constexpr bool gather = false, hside = false, planes3 = true;
};
template <>
struct Traits<Op::Split> {
    static constexpr bool gather = true, hside = false, planes3 = false;
};
template <>
struct Traits<Op::Merge> {
    static constexpr bool gather = false, hside = true, planes3 = false;
};

template <Op OP, int VB, bool CONTIG>
__global__ __launch_bounds__(kThreads) void relayout_kernel(const KernelArgs a)
{
    using Tr = Traits<OP>;
    using V = typename Vec<VB>::type;
    constexpr int VE = VB / 2;  // BF16 elements per vector

    // Workgroup -> (rank, chunk, plane, tile).
    const uint32_t wg = blockIdx.x;
    uint32_t plane = 0, tile, rest;
    int32_t c;
    int64_t p;
    if (VRL_RANK_INNER && Tr::hside) {
        // Pack and merge: the P head groups of one token row belong to
        // different ranks, so the rank varies fastest and neighbouring
        // workgroups cover whole rows of the [S_l][H][D] side together.
        p = int64_t(wg % uint32_t(a.P));
        rest = wg / uint32_t(a.P);
        if (Tr::planes3 && VRL_PLANE_INNER) {
            // ... and the plane next, so that the workgroups in flight read
            // whole fused Q|K|V rows of the source.
            plane = rest % 3u;
            rest /= 3u;
            tile = rest % a.tiles;
            rest /= a.tiles;
        } else {
            tile = rest % a.tiles;
            rest /= a.tiles;
            if (Tr::planes3) {
                plane = rest % 3u;
                rest /= 3u;
            }
        }
        c = a.c_begin + int32_t(rest);
    } else {
        // Unpack and split: one rank's blocks are one contiguous token range
        // of the [S][G][D] side; blocks run in wire-buffer order.
        const uint32_t blk = wg / a.tiles;
        tile = wg - blk * a.tiles;
        rest = blk;
        if (Tr::planes3) {
            plane = rest % 3u;
            rest /= 3u;
        }
        c = a.c_begin + int32_t(rest % uint32_t(a.n_win));
        p = int64_t(rest / uint32_t(a.n_win));
    }
    const int64_t T = a.chunk_q + (c < a.chunk_r ? 1 : 0);
    const int64_t off = int64_t(c) * a.chunk_q + (c < a.chunk_r ? c : a.chunk_r);
    const uint32_t nvec = uint32_t(T) * a.row_vecs;
    const uint32_t f0 = tile * kTileVecs;
    if (f0 >= nvec)
        return;

    const int64_t GD = int64_t(a.G) * a.D;
    const int64_t wire_row0 =
        Tr::planes3 ? p * 3 * a.s_local + 3 * off + int64_t(plane) * T : p * a.s_local + off;
    const int64_t tok0 = Tr::hside ? off : p * a.s_local + off;
    const int64_t head0 = Tr::hside ? p * a.G : 0;
    const int64_t st = a.view_st[plane], sh = a.view_sh[plane];

    uint16_t *const view = a.view_ptr[plane] + tok0 * st + head0 * sh;
    uint16_t *const wire = a.wire + wire_row0 * GD;

    // View-side element offset of vector f of the block.
    auto view_off = [&](uint32_t f) -> int64_t {
        const uint32_t r = div_magic(f, a.row_magic, a.row_shift);
        const uint32_t j = f - r * a.row_vecs;
        if (CONTIG)
            return int64_t(r) * st + int64_t(j) * VE;
        const uint32_t h = div_magic(j, a.head_magic, a.head_shift);
        const uint32_t e = j - h * a.head_vecs;
        return int64_t(r) * st + int64_t(h) * sh + int64_t(e) * VE;
    };
    auto src_of = [&](uint32_t f) -> const V * {
        return Tr::gather ? reinterpret_cast<const V *>(view + view_off(f))
                          : reinterpret_cast<const V *>(wire + int64_t(f) * VE);
    };
    auto dst_of = [&](uint32_t f) -> V * {
        return Tr::gather ? reinterpret_cast<V *>(wire + int64_t(f) * VE)
                          : reinterpret_cast<V *>(view + view_off(f));
    };

    const uint32_t f_lane = f0 + threadIdx.x;
    if (f0 + kTileVecs <= nvec) {
        // Full tile: all loads in flight before the first store.
        V buf[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            buf[u] = load_vec(src_of(f_lane + uint32_t(u * kThreads)));
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            store_vec(dst_of(f_lane + uint32_t(u * kThreads)), buf[u]);
    } else {
        // Last, partial tile of a block.
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t f = f_lane + uint32_t(u * kThreads);
            if (f < nvec)
                store_vec(dst_of(f), load_vec(src_of(f)));
        }
    }
}

template <Op OP, int VB>
hipError_t launch_vb(const LaunchPlan &pl, hipStream_t stream)
{
    const void *fn = pl.contig ? reinterpret_cast<const void *>(&relayout_kernel<OP, VB, true>)
                               : reinterpret_cast<const void *>(&relayout_kernel<OP, VB, false>);
    KernelArgs args = pl.args;
    void *kargs[] = {&args};
    return hipLaunchKernel(fn, dim3(pl.grid), dim3(kThreads), kargs, 0, stream);
}

template <Op OP>
hipError_t launch_op(const LaunchPlan &pl, hipStream_t stream)
{
    switch (pl.vec_bytes) {
    case 16: return launch_vb<OP, 16>(pl, stream);
    case 8: return launch_vb<OP, 8>(pl, stream);
    case 4: return launch_vb<OP, 4>(pl, stream);
    case 2: return launch_vb<OP, 2>(pl, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch(const LaunchPlan &pl, hipStream_t stream)
{
    switch (pl.op) {
    case Op::Pack: return launch_op<Op::Pack>(pl, stream);
    case Op::Unpack: return launch_op<Op::Unpack>(pl, stream);
    case Op::Split: return launch_op<Op::Split>(pl, stream);
    case Op::Merge: return launch_op<Op::Merge>(pl, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace vrl
