// gfx950 kernels of the direct sequence<->head relayout.
//
// All four relayouts (Vflash, "Sol-Engine alignment on SM86 and SM89",
// section "What is enabled": QKV destination pack, attention-result split,
// returned-head merge; plus the receive-side QKV unpack named in the
// performance guide's sequence-head profile) are one batched copy between a
// dense wire block [T][Gb][D] and a strided region of a caller's view:
//
//   wire row (token t of the block)  <->  view row: Gb heads of D elements at
//                                         token tok0 + t, heads head0 ..
//
// With token chunks a block is T(c) tokens of all G heads of a group; with
// head chunks it is all S_l tokens of Gc = G / C heads.
// Pack and merge touch the [S_l][H][D] side (dest/source rank selects the
// head group), unpack and split the [S][G][D] side (rank selects the token
// range).  Pack and split gather view -> wire, unpack and merge scatter
// wire -> view.  Only integer moves: BF16 bit patterns travel in 2..16-byte
// unsigned vectors and never through float registers, so -0, subnormals and
// NaN payloads are preserved.
//
// Mapping to CDNA4.  One workgroup of the direct kernel -- a single wave64
// -- moves one 1 KiB tile of consecutive vectors of one wire block;
// the grid is flattened over (rank, chunk, plane, token tile).  Lanes take
// consecutive 16-byte vectors, so the wave moves 1 KiB per instruction: four
// 128-element head rows, contiguous on the wire side and, for
// head-contiguous views, on the view side as well.  Tiles this small keep
// the chip's in-flight window in address order at fine grain: each wave's
// slot is refilled with the next tile as soon as it is done.  The dense wire
// offset of vector f is f itself; the view offset needs f's row and column,
// obtained with a precomputed multiply-shift division.  Address arithmetic
// is 64-bit wherever a product can pass 2^31 elements.
//
// Views stored head-major, written by a scatter, go through headrun_kernel
// instead (each workgroup moves a run of one head's consecutive tokens), or,
// when head rows are narrower than a cache line, through staged_kernel (an
// LDS transpose of a tile of tokens x heads).
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

// Streaming cache policy: every byte is touched exactly once, so loads and
// stores are non-temporal.
template <typename V>
__device__ __forceinline__ V load_vec(const V *p)
{
    return __builtin_nontemporal_load(p);
}

template <typename V>
__device__ __forceinline__ void store_vec(V *p, V v)
{
    __builtin_nontemporal_store(v, p);
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

// Position of one workgroup: wire block (rank p, chunk c, plane) and the
// tile of that block it moves; plus the block's token count and the base
// pointers of its wire block and of its first view row.
struct Block {
    int64_t T;           // tokens (wire rows) in the block
    uint32_t tile;
    uint32_t plane;
    int64_t st, sh;      // the view's strides for this plane
    uint16_t *view;      // element (first token of the chunk, first head of the group)
    uint16_t *wire;      // first element of the wire block
};

// Wire block (rank p, chunk c, plane): its token count and the base pointers
// of the block and of its first view row.
template <Op OP>
__device__ __forceinline__ Block block_at(const KernelArgs &a, int64_t p, int32_t c, uint32_t plane)
{
    using Tr = Traits<OP>;
    Block b;
    b.tile = 0;
    b.plane = plane;
    const int64_t nq = Tr::planes3 ? 3 : 1;
    const int64_t row = int64_t(a.row_heads) * a.D;  // elements per wire row
    int64_t tok_off, head_off, wire_row0;
    if (a.chunk_heads) {
        // chunk c = heads [c*Gc, (c+1)*Gc) of the group, all S_l tokens
        b.T = a.s_local;
        tok_off = 0;
        head_off = int64_t(c) * a.row_heads;
        wire_row0 = ((p * a.C + c) * nq + plane) * a.s_local;
    } else {
        // chunk c = tokens [off(c), off(c) + T(c)), all G heads
        b.T = a.chunk_q + (c < a.chunk_r ? 1 : 0);
        tok_off = int64_t(c) * a.chunk_q + (c < a.chunk_r ? c : a.chunk_r);
        head_off = 0;
        wire_row0 = p * nq * a.s_local + nq * tok_off + int64_t(plane) * b.T;
    }
    const int64_t tok0 = (Tr::hside ? 0 : p * a.s_local) + tok_off;
    const int64_t head0 = (Tr::hside ? p * a.G : 0) + head_off;
    b.st = a.view_st[plane];
    b.sh = a.view_sh[plane];
    b.view = a.view_ptr[plane] + tok0 * b.st + head0 * b.sh;
    b.wire = a.wire + wire_row0 * row;
    return b;
}

template <Op OP>
__device__ __forceinline__ Block locate(const KernelArgs &a)
{
    using Tr = Traits<OP>;
    const uint32_t wg = blockIdx.x;
    uint32_t plane = 0, tile, rest;
    int32_t c;
    int64_t p;
    if (a.chunk_heads && !Tr::gather) {
        // Scatters with head chunks: a view row is cut into C pieces (and P
        // pieces on the [S_l][H][D] side), so the chunk varies fastest, then
        // the rank, and the pieces of a row are written together.  (Gathers
        // keep the order below: for them this order multiplies the wire
        // streams written at once, and measured slower.)
        c = a.c_begin + int32_t(wg % uint32_t(a.n_win));
        rest = wg / uint32_t(a.n_win);
        if (Tr::hside) {
            p = int64_t(rest % uint32_t(a.P));
            rest /= uint32_t(a.P);
            tile = rest % a.tiles;
            rest /= a.tiles;
            plane = Tr::planes3 ? rest : 0;
        } else {
            tile = rest % a.tiles;
            rest /= a.tiles;
            if (Tr::planes3) {
                plane = rest % 3u;
                rest /= 3u;
            }
            p = int64_t(rest);
        }
    } else if (Tr::hside) {
        // Pack and merge: the P head groups of one token row belong to
        // different ranks, so the rank varies fastest and neighbouring
        // workgroups cover whole rows of the [S_l][H][D] side together.
        p = int64_t(wg % uint32_t(a.P));
        rest = wg / uint32_t(a.P);
        tile = rest % a.tiles;
        rest /= a.tiles;
        if (Tr::planes3) {
            plane = rest % 3u;
            rest /= 3u;
        }
        c = a.c_begin + int32_t(rest);
    } else {
        // Unpack and split: one rank's blocks are one contiguous token range
        // of the [S][G][D] side.  The unpack with token chunks takes the
        // planes one after the other, and within a plane the blocks in token
        // order (chunk fastest, then rank), so consecutive blocks write
        // adjacent rows of one output tensor; otherwise blocks run in
        // wire-buffer order.
        const uint32_t blk = wg / a.tiles;
        tile = wg - blk * a.tiles;
        rest = blk;
        if (Tr::planes3 && !a.chunk_heads) {
            c = a.c_begin + int32_t(rest % uint32_t(a.n_win));
            rest /= uint32_t(a.n_win);
            p = int64_t(rest % uint32_t(a.P));
            plane = rest / uint32_t(a.P);
        } else {
            if (Tr::planes3) {
                plane = rest % 3u;
                rest /= 3u;
            }
            c = a.c_begin + int32_t(rest % uint32_t(a.n_win));
            p = int64_t(rest / uint32_t(a.n_win));
        }
    }
    Block b = block_at<OP>(a, p, c, plane);
    b.tile = tile;
    return b;
}

// Direct kernel: each workgroup moves one 1 KiB tile (kTile consecutive
// vectors) of a wire block; the view side follows.  Used for every call
// except scatters into head-major views.
template <Op OP, int VB, bool CONTIG>
__global__ __launch_bounds__(direct_threads(VB)) void relayout_kernel(const KernelArgs a)
{
    using Tr = Traits<OP>;
    using V = typename Vec<VB>::type;
    constexpr int VE = VB / 2;  // BF16 elements per vector
    constexpr int kLanes = direct_threads(VB);
    constexpr uint32_t kTile = direct_tile_vecs(VB);
    constexpr int kU = int(kTile) / kLanes;  // vectors per lane

    const Block b = locate<OP>(a);
    const uint32_t nvec = uint32_t(b.T) * a.row_vecs;
    const uint32_t f0 = b.tile * kTile;
    if (f0 >= nvec)
        return;
    const int64_t st = b.st, sh = b.sh;
    uint16_t *const view = b.view;
    uint16_t *const wire = b.wire;

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
    if (f0 + kTile <= nvec) {
        // Full tile: all loads in flight before the first store.
        V buf[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            buf[u] = load_vec(src_of(f_lane + uint32_t(u * kLanes)));
#pragma unroll
        for (int u = 0; u < kU; ++u)
            store_vec(dst_of(f_lane + uint32_t(u * kLanes)), buf[u]);
    } else {
        // Last, partial tile of a block.
        for (int u = 0; u < kU; ++u) {
            const uint32_t f = f_lane + uint32_t(u * kLanes);
            if (f < nvec)
                store_vec(dst_of(f), load_vec(src_of(f)));
        }
    }
}

// Workgroup -> (rank p, chunk c, head or head group g, plane) for the
// head-run and staged kernels, after the token tile has been taken off
// `rest`: the workgroups that continue one head-major run come next to each
// other.  For the unpack, which writes the [S][G][D] side, a head's run is
// the whole sequence, rank after rank, so the rank varies right after the
// token tile (with token chunks after the chunk, whose tokens come first
// within a rank): fewer head runs are written at once.  Otherwise the chunk
// follows the token tile and the rank varies slowest: on the [S_l][H][D]
// side each rank has heads of its own, and a gather (split) keeps writing
// one rank's wire block at a time.
template <Op OP>
__device__ __forceinline__ void decode_run(const KernelArgs &a, uint32_t rest, uint32_t groups, int64_t &p,
                                           int32_t &c, uint32_t &g, uint32_t &plane)
{
    using Tr = Traits<OP>;
    plane = 0;
    if (!Tr::hside && !Tr::gather) {
        if (a.chunk_heads) {
            p = int64_t(rest % uint32_t(a.P));
            rest /= uint32_t(a.P);
            c = a.c_begin + int32_t(rest % uint32_t(a.n_win));
            rest /= uint32_t(a.n_win);
        } else {
            c = a.c_begin + int32_t(rest % uint32_t(a.n_win));
            rest /= uint32_t(a.n_win);
            p = int64_t(rest % uint32_t(a.P));
            rest /= uint32_t(a.P);
        }
        g = rest % groups;
        rest /= groups;
        if (Tr::planes3)
            plane = rest;
        return;
    }
    c = a.c_begin + int32_t(rest % uint32_t(a.n_win));
    rest /= uint32_t(a.n_win);
    g = rest % groups;
    rest /= groups;
    if (Tr::planes3) {
        plane = rest % 3u;
        rest /= 3u;
    }
    p = int64_t(rest);
}

// Staged kernel, for head-major views whose head rows (2*D bytes) are
// narrower than a cache line: there the token and head axes swap below line
// granularity, so the swap goes through LDS.  A workgroup takes TT tokens x
// Gt heads of one wire block: for a scatter Gt is the fewest heads (dividing
// the group) whose head rows fill at least one 128-byte line of the wire
// row, for a gather the whole group, so that it writes whole wire rows.  It
// reads the tile in the source's contiguous order into LDS (laid out
// [token][Gt heads]) and after a barrier writes it in the destination's
// contiguous order: runs of TT tokens per head for a scatter, wire-row
// pieces for a gather.  Workgroups are ordered as the head runs are
// (decode_run), token tile fastest.
//
// LDS rows are not padded; instead the column of each vector is XORed with
// a per-token swizzle ((t >> swz_shift) * head_vecs, masked to the largest
// power of two dividing the row, at most one bank sweep of vectors).  The
// view-order phase has a wave's lanes walk one head's column down
// consecutive tokens; the swizzle moves consecutive tokens' head rows onto
// different banks, while the wire-order phase, which walks along rows,
// still sees a permutation of whole aligned groups of columns.
template <Op OP, int VB>
__global__ __launch_bounds__(kStagedThreads) void staged_kernel(const KernelArgs a)
{
    using Tr = Traits<OP>;
    using V = typename Vec<VB>::type;
    constexpr int VE = VB / 2;
    constexpr int kU = Tr::gather ? kGatherUnroll : kScatterUnroll;  // vectors per lane per pass
    constexpr uint32_t kBatch = uint32_t(kStagedThreads) * uint32_t(kU);
    extern __shared__ __align__(16) unsigned char lds_raw[];
    V *const lds = reinterpret_cast<V *>(lds_raw);

    const uint32_t tt_i = blockIdx.x % a.tok_tiles;
    const uint32_t groups = uint32_t(a.row_heads) / a.group_heads;
    int64_t p;
    int32_t c;
    uint32_t hg, plane;
    decode_run<OP>(a, blockIdx.x / a.tok_tiles, groups, p, c, hg, plane);
    const Block b = block_at<OP>(a, p, c, plane);
    const uint32_t TT = a.tile_tokens;
    const uint32_t t0 = tt_i * TT;
    if (int64_t(t0) >= b.T)
        return;
    const uint32_t tte = uint32_t(min(int64_t(TT), b.T - t0));  // tokens in this tile
    const uint32_t hv = a.head_vecs;
    const uint32_t gv = a.group_heads * hv;                        // vectors of a tile row
    const uint32_t nv = TT * gv;                                   // vectors of a full tile
    const int64_t st = b.st, sh = b.sh, row = int64_t(a.row_heads) * a.D;
    const uint32_t h0 = hg * a.group_heads;
    uint16_t *const view = b.view + int64_t(t0) * st + int64_t(h0) * sh;
    uint16_t *const wire = b.wire + int64_t(t0) * row + int64_t(h0) * a.D;

    // Tile element i in wire order: token t, column j = h * hv + e.
    // In view order: head h, token t, column e.
    struct Pos {
        uint32_t t, lds;
        int64_t off;  // element offset on the side being read or written
    };
    // LDS slot of column j of token t (swz_mask + 1 divides gv, so the XOR
    // stays inside the row)
    auto slot = [&](uint32_t t, uint32_t j) -> uint32_t {
        return t * gv + (j ^ (((t >> a.swz_shift) * hv) & a.swz_mask));
    };
    auto wire_order = [&](uint32_t i) -> Pos {
        const uint32_t t = div_magic(i, a.gv_magic, a.gv_shift);
        const uint32_t j = i - t * gv;
        return Pos{t, slot(t, j), int64_t(t) * row + int64_t(j) * VE};
    };
    auto view_order = [&](uint32_t i) -> Pos {
        const uint32_t h = div_magic(i, a.tv_magic, a.tv_shift);
        const uint32_t r = i - h * (TT * hv);
        const uint32_t t = div_magic(r, a.head_magic, a.head_shift);
        const uint32_t e = r - t * hv;
        return Pos{t, slot(t, h * hv + e), int64_t(t) * st + int64_t(h) * sh + int64_t(e) * VE};
    };

    // Phase 1: source -> LDS, in the source's contiguous order.  A scatter
    // loads on every lane, a lane past the tile's end from the tile's first
    // element (which always exists), so that no branch separates its loads:
    // under per-vector branches the compiler waited for the first load
    // before issuing the second.  A gather keeps the branches: its batch is
    // larger than its tile at 16-byte vectors, and the lanes past the tile
    // skip their loads and LDS reads.
    for (uint32_t i0 = 0; i0 < nv; i0 += kBatch) {
        V buf[kU];
        uint32_t slot[kU];
        bool ok[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const uint32_t i = i0 + uint32_t(u * kStagedThreads) + threadIdx.x;
            const Pos q = Tr::gather ? view_order(i < nv ? i : 0) : wire_order(i < nv ? i : 0);
            ok[u] = i < nv && q.t < tte;
            slot[u] = q.lds;
            if constexpr (Tr::gather) {
                if (ok[u])
                    buf[u] = load_vec(reinterpret_cast<const V *>(view + q.off));
            } else {
                buf[u] = load_vec(reinterpret_cast<const V *>(wire + (ok[u] ? q.off : 0)));
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (ok[u])
                lds[slot[u]] = buf[u];
    }
    __syncthreads();
    // Phase 2: LDS -> destination, in the destination's contiguous order (all
    // LDS reads of a batch first, then the stores; as in phase 1 a scatter
    // reads on every lane, slot 0 standing in past the tile's end).
    for (uint32_t i0 = 0; i0 < nv; i0 += kBatch) {
        V buf[kU];
        int64_t doff[kU];
        bool ok[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const uint32_t i = i0 + uint32_t(u * kStagedThreads) + threadIdx.x;
            const Pos q = Tr::gather ? wire_order(i < nv ? i : 0) : view_order(i < nv ? i : 0);
            ok[u] = i < nv && q.t < tte;
            doff[u] = q.off;
            if constexpr (Tr::gather) {
                if (ok[u])
                    buf[u] = lds[q.lds];
            } else {
                buf[u] = lds[ok[u] ? q.lds : 0u];
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (ok[u])
                store_vec(reinterpret_cast<V *>((Tr::gather ? wire : view) + doff[u]), buf[u]);
    }
}

// Head-run kernel, for views stored head-major: a workgroup moves TT
// consecutive tokens of one head of a wire block (TT * head_vecs <= headrun_tile_vecs(VB)
// vectors), and consecutive workgroups take consecutive token tiles of the
// same head.  The head-major side then sees one contiguous run per
// workgroup and the chip writes (or reads) few runs at a time; the wire side
// sees TT pieces of D elements, one per wire row.
template <Op OP, int VB>
__global__ __launch_bounds__(kHeadrunThreads) void headrun_kernel(const KernelArgs a)
{
    using Tr = Traits<OP>;
    using V = typename Vec<VB>::type;
    constexpr int VE = VB / 2;
    constexpr uint32_t kTile = headrun_tile_vecs(VB);
    constexpr int kU = int(kTile) / kHeadrunThreads;  // vectors per lane

    // token tile fastest, then what continues the same head's run
    const uint32_t tt_i = blockIdx.x % a.tok_tiles;
    int64_t p;
    int32_t c;
    uint32_t h, plane;
    decode_run<OP>(a, blockIdx.x / a.tok_tiles, uint32_t(a.row_heads), p, c, h, plane);
    const Block b = block_at<OP>(a, p, c, plane);
    const uint32_t t0 = tt_i * a.tile_tokens;
    if (int64_t(t0) >= b.T)
        return;
    const uint32_t tte = uint32_t(min(int64_t(a.tile_tokens), b.T - t0));
    const uint32_t nv = tte * a.head_vecs;  // vectors of this tile
    const int64_t st = b.st, row = int64_t(a.row_heads) * a.D;
    uint16_t *const view = b.view + int64_t(t0) * st + int64_t(h) * b.sh;
    uint16_t *const wire = b.wire + int64_t(t0) * row + int64_t(h) * a.D;

    // element offset of vector i (token t, column e) on a side whose token stride is `stride`
    auto off = [&](uint32_t i, int64_t stride) -> int64_t {
        const uint32_t t = div_magic(i, a.head_magic, a.head_shift);
        return int64_t(t) * stride + int64_t(i - t * a.head_vecs) * VE;
    };
    auto src_of = [&](uint32_t i) -> const V * {
        return reinterpret_cast<const V *>(Tr::gather ? view + off(i, st) : wire + off(i, row));
    };
    auto dst_of = [&](uint32_t i) -> V * {
        return reinterpret_cast<V *>(Tr::gather ? wire + off(i, row) : view + off(i, st));
    };

    if (nv == kTile) {
        V buf[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            buf[u] = load_vec(src_of(threadIdx.x + uint32_t(u * kHeadrunThreads)));
#pragma unroll
        for (int u = 0; u < kU; ++u)
            store_vec(dst_of(threadIdx.x + uint32_t(u * kHeadrunThreads)), buf[u]);
    } else {
        for (int u = 0; u < kU; ++u) {
            const uint32_t i = threadIdx.x + uint32_t(u * kHeadrunThreads);
            if (i < nv)
                store_vec(dst_of(i), load_vec(src_of(i)));
        }
    }
}

template <Op OP, int VB>
hipError_t launch_vb(const LaunchPlan &pl, hipStream_t stream)
{
    KernelArgs args = pl.args;
    void *kargs[] = {&args};
    if (pl.headrun)
        return hipLaunchKernel(reinterpret_cast<const void *>(&headrun_kernel<OP, VB>), dim3(pl.grid),
                               dim3(kHeadrunThreads), kargs, 0, stream);
    if (pl.lds_bytes)
        return hipLaunchKernel(reinterpret_cast<const void *>(&staged_kernel<OP, VB>), dim3(pl.grid),
                               dim3(kStagedThreads), kargs, pl.lds_bytes, stream);
    const void *fn = pl.contig ? reinterpret_cast<const void *>(&relayout_kernel<OP, VB, true>)
                               : reinterpret_cast<const void *>(&relayout_kernel<OP, VB, false>);
    return hipLaunchKernel(fn, dim3(pl.grid), dim3(direct_threads(VB)), kargs, 0, stream);
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
