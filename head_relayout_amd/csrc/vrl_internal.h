// Internal interface between the C-ABI layer (vrl_api.cpp) and the gfx950
// kernels (vrl_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace vrl {

// Workgroup shapes.  The direct and head-run kernels move one tile per
// workgroup, each lane issuing its loads before its stores; the staged
// kernel moves its LDS tile in batches.  The direct kernel runs one wave per
// workgroup on 1 KiB tiles (one 16-byte vector per lane): tiles dispatched
// in address order, each workgroup's slot refilled as soon as its one wave
// is done.  The head-run kernel takes 128 lanes on 4 KiB tiles (16 tokens of
// a 128-element head at 16-byte vectors); the LDS transpose needs its 256
// lanes to fill and drain a tile.  Tile sizes are in bytes, so narrow
// vectors keep the same tiles.
constexpr int kDirectThreads = 64;
constexpr uint32_t kDirectTileBytes = 1024;
// Narrower vectors (operands not 16-byte aligned) move less per wave
// instruction and do better with 256 lanes on 4 KiB tiles.
constexpr int kNarrowThreads = 256;
constexpr uint32_t kNarrowTileBytes = 4096;
constexpr int kHeadrunThreads = 128;
constexpr uint32_t kHeadrunTileBytes = 4096;
constexpr int kStagedThreads = 256;
// The staged kernel's LDS tile and batch (vectors per lane per pass): 8 KiB
// tiles moved 512 vectors at a time for scatters, 16 KiB tiles of whole wire
// rows moved 2,048 at a time for gathers.
constexpr uint32_t kScatterLdsBytes = 8192;
constexpr int kScatterUnroll = 2;
constexpr uint32_t kGatherLdsBytes = 16384;
constexpr int kGatherUnroll = 8;
constexpr uint32_t kStagedBatch = uint32_t(kStagedThreads) * uint32_t(kGatherUnroll);  // the larger batch
// Lanes and vectors per tile of the direct kernel at a vector width of vb
// bytes; vectors per tile of the head-run kernel.
constexpr int direct_threads(int vb) { return vb == 16 ? kDirectThreads : kNarrowThreads; }
constexpr uint32_t direct_tile_vecs(int vb) { return (vb == 16 ? kDirectTileBytes : kNarrowTileBytes) / uint32_t(vb); }
constexpr uint32_t headrun_tile_vecs(int vb) { return kHeadrunTileBytes / uint32_t(vb); }
// Bound on any tile or batch in vectors (2-byte vectors), for the planner's
// index-range checks.
constexpr uint32_t kMaxTileVecs = kStagedBatch > kHeadrunTileBytes / 2 ? kStagedBatch : kHeadrunTileBytes / 2;

// Head-major views (a head's tokens closer together than a token's heads)
// whose head rows (2*D bytes) are narrower than this go through the LDS
// transpose (staged_kernel); scatters into head-major views with wider head
// rows run as head runs (headrun_kernel), gathers from them in wire order.
constexpr int64_t kHeadrunMinBytes = 128;

enum class Op : int { Pack = 0, Unpack = 1, Split = 2, Merge = 3 };

// Everything a kernel needs, passed by value as the kernel argument.
// "view" is the strided side (the caller's [rows][heads][D] tensors), "wire"
// the dense exchange buffer.  Strides are in elements.
struct KernelArgs {
    uint16_t *view_ptr[3];  // per plane q/k/v (one used by split and merge)
    int64_t view_st[3];     // token-axis stride
    int64_t view_sh[3];     // head-axis stride
    uint16_t *wire;
    int64_t s_local;
    int32_t P, G, D;
    int32_t C;
    int32_t chunk_heads;       // chunks split head groups instead of tokens
    int32_t row_heads;         // heads per wire row: G, or G / C with chunk_heads
    int32_t chunk_q, chunk_r;  // S_l / C and S_l % C
    int32_t c_begin, n_win;    // chunk window [c_begin, c_begin + n_win)
    uint32_t tiles;            // workgroups per wire block
    uint32_t row_vecs;         // vectors per wire row (one token's G heads)
    uint32_t head_vecs;        // vectors per head row (D elements)
    uint32_t row_shift;        // f / row_vecs == (f * row_magic) >> row_shift
    uint64_t row_magic;
    uint64_t head_magic;       // j / head_vecs, same scheme
    uint32_t head_shift;
    uint32_t tile_tokens;      // head-run and staged kernels: tokens per tile (TT)
    uint32_t tok_tiles;        // head-run and staged kernels: token tiles per block
    uint32_t group_heads;      // staged kernel: heads per tile (Gt, divides row_heads)
    uint32_t gv_shift;
    uint64_t gv_magic;         // staged kernel: i / (Gt * head_vecs)
    uint64_t tv_magic;         // staged kernel: i / (TT * head_vecs)
    uint32_t tv_shift;
    uint32_t swz_shift;        // staged kernel: LDS column swizzle of token t is
    uint32_t swz_mask;         //   ((t >> swz_shift) * head_vecs) & swz_mask
};

struct LaunchPlan {
    Op op;
    int vec_bytes;     // 16, 8, 4 or 2
    bool contig;       // every view row's G heads are one contiguous run
    bool headrun;      // head-major view: runs of one head's tokens (headrun_kernel)
    uint32_t lds_bytes;  // nonzero: head-major view through the LDS transpose (staged_kernel)
    uint32_t grid;     // workgroups
    KernelArgs args;
};

// Problem size (the C ABI's vrl_dims) and one operand view, as the planner
// sees them: byte address and element strides.
struct Problem {
    int32_t P, C;
    int64_t s_local;
    int32_t H, D;
    int32_t chunk_heads;
};
struct PlanView {
    uintptr_t ptr;
    int64_t st, sh;
};

// Plans a launch (vrl_plan.cpp).  Returns false, with *why set, when the
// problem exceeds what one launch can index.
bool plan_launch(Op op, const Problem &pb, const PlanView *views, int nviews, uintptr_t wire,
                 int32_t c_begin, int32_t c_end, LaunchPlan &pl, const char **why);

// Enqueues the planned kernel on `stream`; returns the launch status.
hipError_t launch(const LaunchPlan &plan, hipStream_t stream);

}  // namespace vrl
