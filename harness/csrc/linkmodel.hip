// Link-paced exchange for P virtual ranks held in one GPU.
//
// Stand-in for the all-to-all of a sequence-parallel attention layer (the
// collective the Vflash performance guide's profile of one denoising request
// runs on a side stream, where it may overlap the pack or the attention):
// every (sender, receiver) block is copied inside the one HBM, and a block
// that would cross an inter-GPU link is paced to that link's rate.  Each
// pair of distinct ranks has a link of its own (a full mesh, as xGMI on an
// eight-GPU MI355X node), so all paced blocks run at once, each at the link
// rate; a rank's block to itself is a local copy and runs unpaced.  The
// bytes move for real, so a schedule built on it computes the same buffers
// as one with an unpaced exchange, while the HBM sees only the traffic the
// links would carry.
//
// Test and benchmark infrastructure only; the relayout library does not use
// it.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kMaxBlocks = 64;
// Workgroups sharing one block: one per kGbsPerGroup of link rate, within
// [kMinGroups, kMaxGroups].  A workgroup keeps one 32 KiB piece in flight
// and copies about 7 GB/s on its own, so each paced one is asked for less
// than half of that.
constexpr double kGbsPerGroup = 3.0;
constexpr uint32_t kMinGroups = 8, kMaxGroups = 128;

struct Block {
    const void *src;
    void *dst;
    uint64_t bytes;
    uint32_t paced;
    uint32_t pad_;
};

struct Args {
    Block blk[kMaxBlocks];
    int32_t nblocks;
    uint32_t groups;           // workgroups per block
    uint64_t ticks_per_piece;  // wall-clock ticks one workgroup spends on a piece of a paced block
    uint64_t max_spins;        // bound on every workgroup's waiting
};

template <int VB>
struct Vec;
template <>
struct Vec<16> {
    typedef uint32_t type __attribute__((ext_vector_type(4)));
};
template <>
struct Vec<2> {
    typedef uint16_t type;
};

// Workgroup g of block b copies pieces g, g + groups, ... of the block (a
// piece is kThreads * kUnroll vectors).  On a paced block the k-th piece a
// workgroup copies may start no earlier than k * ticks_per_piece after the
// workgroup began, so the block's groups together move it at the link rate.
// The wait ends when the clock passes that time or after max_spins sleeps,
// whichever comes first.
template <int VB>
__global__ __launch_bounds__(kThreads) void paced_copy(const Args a)
{
    using V = typename Vec<VB>::type;
    const uint32_t b = blockIdx.x / a.groups;
    const uint32_t g = blockIdx.x - b * a.groups;
    if (b >= uint32_t(a.nblocks))
        return;
    const Block blk = a.blk[b];
    const uint64_t nvec = blk.bytes / VB;
    constexpr uint64_t piece = uint64_t(kThreads) * kUnroll;
    const uint64_t npieces = (nvec + piece - 1) / piece;
    const V *src = static_cast<const V *>(blk.src);
    V *dst = static_cast<V *>(blk.dst);
    const uint64_t t0 = wall_clock64();
    uint64_t spins = 0, k = 0;
    for (uint64_t pc = g; pc < npieces; pc += a.groups, ++k) {
        if (blk.paced) {
            const uint64_t due = t0 + k * a.ticks_per_piece;
            while (uint64_t(wall_clock64()) < due && spins < a.max_spins) {
                __builtin_amdgcn_s_sleep(2);
                ++spins;
            }
        }
        const uint64_t f0 = pc * piece + threadIdx.x;
        V buf[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t f = f0 + uint64_t(u) * kThreads;
            if (f < nvec)
                buf[u] = __builtin_nontemporal_load(src + f);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t f = f0 + uint64_t(u) * kThreads;
            if (f < nvec)
                __builtin_nontemporal_store(buf[u], dst + f);
        }
    }
}

thread_local char g_err[256];

int fail(const char *msg)
{
    std::snprintf(g_err, sizeof g_err, "%s", msg);
    return 1;
}

}  // namespace

extern "C" {

// One exchanged block: `bytes` bytes from `src` to `dst` (device memory of
// the current device, not overlapping), paced to the link rate if `paced`.
typedef struct {
    const void *src;
    void *dst;
    uint64_t bytes;
    int32_t paced;
} lm_block;

// Enqueues one exchange of `n` blocks (1 <= n <= 64) on `stream` (a
// hipStream_t, NULL for the default stream): one kernel, 8 to 128
// workgroups per block (one per 3 GB/s of link rate), paced blocks at
// `link_gbs` 1e9 B/s each (1 <= link_gbs <= 10000).
// Returns 0, or 1 with a message from lm_last_error() and nothing enqueued.
__attribute__((visibility("default"))) int lm_exchange(const lm_block *blocks, int32_t n, double link_gbs,
                                                       void *stream)
{
    if (!blocks || n < 1 || n > kMaxBlocks)
        return fail("need 1 to 64 blocks");
    if (!(link_gbs >= 1.0 && link_gbs <= 10000.0))
        return fail("link rate must lie in [1, 10000] GB/s");
    Args a{};
    bool narrow = false;
    double longest = 0;
    for (int i = 0; i < n; ++i) {
        const lm_block &x = blocks[i];
        if (!x.src || !x.dst || x.bytes == 0)
            return fail("a block has a null pointer or no bytes");
        if ((uintptr_t(x.src) | uintptr_t(x.dst) | x.bytes) % 2)
            return fail("blocks must be 2-byte aligned and hold whole 2-byte elements");
        if ((uintptr_t(x.src) | uintptr_t(x.dst) | x.bytes) % 16)
            narrow = true;
        const uintptr_t s = uintptr_t(x.src), d = uintptr_t(x.dst);
        if (s < d + x.bytes && d < s + x.bytes)
            return fail("a block's source and destination overlap");
        a.blk[i] = Block{x.src, x.dst, x.bytes, uint32_t(x.paced != 0), 0};
        if (x.paced && double(x.bytes) > longest)
            longest = double(x.bytes);
    }
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
        return fail("cannot read the device's wall-clock rate");
    const double secs = longest / (link_gbs * 1e9);
    if (secs > 1.0)
        return fail("a paced block would take longer than one second");
    const int vb = narrow ? 2 : 16;
    const double piece_bytes = double(kThreads) * kUnroll * vb;
    uint32_t groups = uint32_t(link_gbs / kGbsPerGroup + 0.999);
    groups = groups < kMinGroups ? kMinGroups : groups > kMaxGroups ? kMaxGroups : groups;
    a.nblocks = n;
    a.groups = groups;
    a.ticks_per_piece = uint64_t(piece_bytes * groups / (link_gbs * 1e9) * khz * 1e3);
    // a sleep lasts at least about 50 ns; allow ten times the paced time's worth
    a.max_spins = uint64_t(secs * 1e9 / 5.0) + 100000;
    void *kargs[] = {&a};
    const void *fn = narrow ? reinterpret_cast<const void *>(&paced_copy<2>)
                            : reinterpret_cast<const void *>(&paced_copy<16>);
    const hipError_t e = hipLaunchKernel(fn, dim3(uint32_t(n) * groups), dim3(kThreads), kargs, 0,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(hipGetErrorString(e));
    return 0;
}

__attribute__((visibility("default"))) const char *lm_last_error(void)
{
    return g_err;
}

}  // extern "C"
