// Random and extreme arguments through the C ABI's host-side validation and
// launch planning, built with AddressSanitizer and UndefinedBehaviorSanitizer
// (g++, host code only).  The few HIP runtime calls the validation makes are
// stubbed here by a fake device -- sometimes missing, sometimes not a gfx950,
// sometimes a gfx950 owning one 16 GiB allocation at 2^40 -- and the kernel
// launch by a stub that records the plan, so no GPU is needed and nothing
// runs on one.
//
// Checks: every call returns a documented status and records a reason on
// error; calls with in-contract views inside the fake allocation on the fake
// gfx950 are accepted and planned with a sane grid; no sanitizer report
// (signed overflow in the size and overlap arithmetic included).
// Prints one summary line; exits 0 when every check holds.
#include "../../include/vrl.h"
#include "../../head_relayout_amd/csrc/vrl_internal.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <utility>

namespace {

uint64_t rng_state = 0x243F6A8885A308D3ull;

uint64_t next()  // SplitMix64
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int64_t below(int64_t n)
{
    return int64_t(next() % uint64_t(n));
}

// The fake device.
enum Mode { NO_DEVICE, OTHER_ARCH, GFX950, BAD_ORDINAL };
Mode g_mode = NO_DEVICE;
constexpr uintptr_t kBase = uintptr_t(1) << 40;
constexpr size_t kSize = size_t(1) << 34;
bool g_foreign = false;  // the allocation belongs to another device
int g_launches = 0;
bool g_launch_bad = false;

}  // namespace

extern "C" {

hipError_t hipGetDevice(int *dev)
{
    switch (g_mode) {
    case NO_DEVICE: return hipErrorNoDevice;
    case OTHER_ARCH: *dev = 1; return hipSuccess;
    case GFX950: *dev = 0; return hipSuccess;
    case BAD_ORDINAL: *dev = 300; return hipSuccess;
    }
    return hipErrorNoDevice;
}

hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *prop, int dev)
{
    std::memset(prop, 0, sizeof *prop);
    std::strcpy(prop->gcnArchName, dev == 0 ? "gfx950:sramecc+:xnack-" : "gfx942:sramecc+:xnack-");
    return hipSuccess;
}

hipError_t hipGetLastError(void)
{
    return hipSuccess;
}

const char *hipGetErrorString(hipError_t)
{
    return "stubbed HIP error";
}

hipError_t hipPointerGetAttributes(hipPointerAttribute_t *attr, const void *p)
{
    const uintptr_t u = reinterpret_cast<uintptr_t>(p);
    if (u < kBase || u >= kBase + kSize)
        return hipErrorInvalidValue;
    std::memset(attr, 0, sizeof *attr);
    attr->type = hipMemoryTypeDevice;
    attr->device = g_foreign ? 1 : 0;
    return hipSuccess;
}

// Fake streams: kStream0 belongs to device 0, kStream1 to device 1, any
// other non-null handle is unknown.
void *const kStream0 = reinterpret_cast<void *>(uintptr_t(0x5000));
void *const kStream1 = reinterpret_cast<void *>(uintptr_t(0x5100));

hipError_t hipStreamGetDevice(hipStream_t stream, hipDevice_t *device)
{
    if (reinterpret_cast<void *>(stream) == kStream0) {
        *device = 0;
        return hipSuccess;
    }
    if (reinterpret_cast<void *>(stream) == kStream1) {
        *device = 1;
        return hipSuccess;
    }
    return hipErrorInvalidHandle;
}

hipError_t hipMemGetAddressRange(hipDeviceptr_t *base, size_t *size, hipDeviceptr_t p)
{
    const uintptr_t u = reinterpret_cast<uintptr_t>(p);
    if (u < kBase || u >= kBase + kSize)
        return hipErrorInvalidValue;
    *base = reinterpret_cast<hipDeviceptr_t>(kBase);
    *size = kSize;
    return hipSuccess;
}

}  // extern "C"

namespace vrl {
hipError_t launch(const LaunchPlan &pl, hipStream_t)
{
    ++g_launches;
    if (pl.grid < 1 || pl.grid >= (uint32_t(1) << 31) ||
        !(pl.vec_bytes == 2 || pl.vec_bytes == 4 || pl.vec_bytes == 8 || pl.vec_bytes == 16) ||
        pl.lds_bytes > kGatherLdsBytes || pl.args.tiles < 1)
        g_launch_bad = true;
    return hipSuccess;
}
}  // namespace vrl

namespace {

int64_t wild64(int64_t small)
{
    switch (next() % 9) {
    case 0: return 0;
    case 1: return -1 - below(5);
    case 2: return std::numeric_limits<int64_t>::max() - below(3);
    case 3: return std::numeric_limits<int64_t>::min() + below(3);
    case 4: return int64_t(next() >> 1);
    case 5: return (int64_t(1) << (16 + below(40))) + below(3) - 1;
    default: return 1 + below(small);
    }
}

int32_t wild32(int32_t small)
{
    switch (next() % 8) {
    case 0: return 0;
    case 1: return -1 - int32_t(below(5));
    case 2: return std::numeric_limits<int32_t>::max() - int32_t(below(3));
    case 3: return std::numeric_limits<int32_t>::min();
    case 4: return int32_t(1) << (8 + below(23));
    default: return 1 + int32_t(below(small));
    }
}

void *wild_ptr()
{
    uintptr_t u;
    switch (next() % 8) {
    case 0: return nullptr;
    case 1: u = 1 + 2 * uintptr_t(below(1024)); break;                       // odd, low
    case 2: u = ~uintptr_t(0) - 16 * uintptr_t(below(4096)) - 1; break;      // top of the address space
    case 3: u = (uintptr_t(1) << 63) - 16 * uintptr_t(below(64)) + 16 * uintptr_t(below(64)); break;
    case 4: u = kBase + kSize - 16 * uintptr_t(below(64)); break;            // end of the allocation
    default: u = kBase + 16 * uintptr_t(below(1 << 20)); break;              // inside it
    }
    return reinterpret_cast<void *>(u);
}

vrl_view wild_view()
{
    return vrl_view{wild_ptr(), wild64(1 << 14), wild64(1 << 14)};
}

// In-contract arguments for `op` (0 pack, 1 unpack, 2 split, 3 merge):
// token-major or head-major views each in its own 1 GiB slot of the fake
// allocation, or column views of one fused row buffer in any column order;
// rows optionally padded; a dense wire buffer in a slot of its own.
struct Args {
    vrl_view v[3];
    void *wire;
};

Args valid_args(int op, const vrl_dims &d)
{
    const bool hside = op == 0 || op == 3;
    const int64_t rows = hside ? d.s_local : int64_t(d.P) * d.s_local;
    const int64_t heads = hside ? d.H : d.H / d.P;
    const int64_t pad = below(3) == 0 ? below(9) : 0;
    const int layout = int(below(3));  // token-major, head-major, fused columns
    Args a;
    const int64_t W = heads * d.D;
    const int perm = int(below(6));     // column order of the fused views
    const int col[6][3] = {{0, 1, 2}, {0, 2, 1}, {1, 0, 2}, {1, 2, 0}, {2, 0, 1}, {2, 1, 0}};
    for (int i = 0; i < 3; ++i) {
        void *p = reinterpret_cast<void *>(kBase + (uintptr_t(i) << 30) + 2 * uintptr_t(below(64)));
        if (layout == 1)
            a.v[i] = vrl_view{p, d.D + pad, rows * (d.D + pad)};
        else if (layout == 0)
            a.v[i] = vrl_view{p, heads * d.D + pad, d.D};
        else
            a.v[i] = vrl_view{reinterpret_cast<void *>(kBase + 2 * uintptr_t(col[perm][i] * W)), 3 * W + pad, d.D};
    }
    a.wire = reinterpret_cast<void *>(kBase + (uintptr_t(3) << 30) + 2 * uintptr_t(below(64)));
    return a;
}

vrl_status call(int op, const vrl_dims *d, Args &a, int32_t cb, int32_t ce, void *stream = nullptr)
{
    switch (op) {
    case 0: return vrl_qkv_pack(d, &a.v[0], &a.v[1], &a.v[2], a.wire, cb, ce, stream);
    case 1: return vrl_qkv_unpack(d, a.wire, &a.v[0], &a.v[1], &a.v[2], cb, ce, stream);
    case 2: return vrl_attn_split(d, &a.v[0], a.wire, cb, ce, stream);
    default: return vrl_head_merge(d, a.wire, &a.v[0], cb, ce, stream);
    }
}

}  // namespace

int main()
{
    const int iters = 300000;
    int bad = 0, accepted = 0, valid_calls = 0;
    auto report = [&](int it, const char *what, int op, vrl_status s) {
        if (bad < 10)
            std::printf("iteration %d op %d: %s (status %d: %s)\n", it, op, what, int(s), vrl_last_error());
        ++bad;
    };
    for (int it = 0; it < iters; ++it) {
        g_mode = Mode(below(4));
        g_foreign = below(8) == 0;
        vrl_dims d{wild32(8), wild32(8), wild64(96), wild32(64), wild32(256), int32_t(below(4)) - 1};
        const bool sane = below(2) == 0;
        if (sane) {
            d.P = 1 + int32_t(below(4));
            d.chunk_heads = int32_t(below(3) == 0);
            d.C = 1 + int32_t(below(4));
            d.H = d.P * d.C * (1 + int32_t(below(6)));
            d.s_local = d.C + below(96);
            d.D = below(4) == 0 ? 1 + int32_t(below(300)) : 8 << below(5);
        }
        const int op = int(below(4));
        const bool valid_layout = sane && below(2) == 0;
        Args a;
        if (valid_layout) {
            a = valid_args(op, d);
        } else {
            for (vrl_view &v : a.v)
                v = wild_view();
            a.wire = wild_ptr();
        }
        int32_t cb, ce;
        if (sane && below(4) != 0) {
            cb = int32_t(below(d.C));
            ce = cb + 1 + int32_t(below(d.C - cb));
        } else {
            cb = int32_t(below(7)) - 1;
            ce = int32_t(below(7)) - 1;
        }
        // mostly the null stream; sometimes a stream of the current device, of
        // another device, or an unknown handle
        const uint64_t sk = below(16);
        void *const stream = sk < 12 ? nullptr : sk < 14 ? kStream0 : sk < 15 ? kStream1
                                                 : reinterpret_cast<void *>(uintptr_t(0x5200));
        const bool stream_ok = stream == nullptr || stream == kStream0;
        const int before = g_launches;
        const vrl_status s = call(op, &d, a, cb, ce, stream);
        const bool launched = g_launches != before;
        if (s == VRL_OK) {
            ++accepted;
            if (!launched)
                report(it, "accepted without a launch", op, s);
            if (g_mode != GFX950 || g_foreign)
                report(it, "accepted without a gfx950 owning the memory", op, s);
            if (!stream_ok)
                report(it, "accepted with another device's or an unknown stream", op, s);
        } else {
            if (launched)
                report(it, "launched but reported an error", op, s);
            if (s != VRL_E_INVALID && s != VRL_E_LAYOUT && s != VRL_E_DEVICE)
                report(it, "undocumented status", op, s);
            if (!vrl_last_error()[0])
                report(it, "error without a reason", op, s);
        }
        const bool window_ok = cb >= 0 && cb < ce && ce <= d.C;
        if (valid_layout && window_ok && g_mode == GFX950 && !g_foreign) {
            ++valid_calls;
            if (stream_ok && s != VRL_OK)
                report(it, "in-contract call rejected", op, s);
            if (!stream_ok && s != VRL_E_DEVICE)
                report(it, "stream of another device not refused as a device error", op, s);
        }
        // the sizing helpers: -1 exactly when a reason is recorded
        if ((vrl_exchange_elems(int(below(3)) - 1, &d) < 0) != (vrl_last_error()[0] != 0))
            report(it, "exchange_elems result and reason disagree", -1, VRL_OK);
        for (int32_t c = -1; c <= 5; ++c)
            if ((vrl_chunk_offset(&d, c) < 0) != (vrl_last_error()[0] != 0))
                report(it, "chunk_offset result and reason disagree", -1, VRL_OK);
        (void)vrl_status_string(vrl_status(int(below(6)) - 1));
    }
    if (g_launch_bad) {
        std::printf("a launch plan had an out-of-range grid, vector width or LDS size\n");
        ++bad;
    }
    // Output views with equal strides placed across 2^63 and at the top of
    // the address space: the overlap test's pointer differences and the
    // views' byte spans must neither overflow nor wrap.
    {
        g_mode = GFX950;
        g_foreign = false;
        const vrl_dims d{2, 2, 8, 4, 16, 0};
        const uintptr_t bases[] = {uintptr_t(1) << 63, ~uintptr_t(0) - 255, uintptr_t(1) << 62};
        for (uintptr_t b : bases)
            for (uintptr_t shift : {uintptr_t(64), uintptr_t(1) << 40})
                for (int op = 0; op < 4; ++op) {
                    Args a;
                    for (int i = 0; i < 3; ++i)
                        a.v[i] = vrl_view{reinterpret_cast<void *>(b - shift + uintptr_t(i) * shift), 2 * 16, 16};
                    a.wire = reinterpret_cast<void *>(b + 3 * shift);
                    const vrl_status s = call(op, &d, a, 0, 2);
                    if (s == VRL_OK)
                        report(-1, "views outside any allocation accepted", op, s);
                }
    }
    // Unpack into fused-row column views that overlap by 1 .. W-1 elements
    // (in either order) must be refused as a layout error; apart by W, accepted.
    for (int it = 0; it < 2000; ++it) {
        g_mode = GFX950;
        g_foreign = false;
        const vrl_dims d{2, 2, 6 + below(8), 4, int32_t(1 + below(40)), 0};
        const int64_t W = int64_t(d.H / d.P) * d.D, gap = 1 + below(W);
        Args a;
        const uintptr_t b0 = kBase + 4096;
        const int first = int(below(3)), second = (first + 1 + int(below(2))) % 3, third = 3 - first - second;
        a.v[first] = vrl_view{reinterpret_cast<void *>(b0), 3 * W, d.D};
        a.v[second] = vrl_view{reinterpret_cast<void *>(b0 + 2 * uintptr_t(gap)), 3 * W, d.D};
        a.v[third] = vrl_view{reinterpret_cast<void *>(b0 + 2 * uintptr_t(gap + W)), 3 * W, d.D};
        if (below(2))  // the same views listed in the other order
            std::swap(a.v[first], a.v[second]);
        a.wire = reinterpret_cast<void *>(kBase + (uintptr_t(3) << 30));
        const vrl_status s = call(1, &d, a, 0, 2);
        if (gap < W && s != VRL_E_LAYOUT)
            report(it, "overlapping fused columns not refused", 1, s);
        if (gap == W && s != VRL_OK)
            report(it, "adjacent fused columns refused", 1, s);
    }
    vrl_view z{nullptr, 0, 0};
    if (vrl_qkv_pack(nullptr, &z, &z, &z, nullptr, 0, 1, nullptr) != VRL_E_INVALID ||
        vrl_qkv_unpack(nullptr, nullptr, &z, &z, &z, 0, 1, nullptr) != VRL_E_INVALID ||
        vrl_attn_split(nullptr, &z, nullptr, 0, 1, nullptr) != VRL_E_INVALID ||
        vrl_head_merge(nullptr, nullptr, &z, 0, 1, nullptr) != VRL_E_INVALID ||
        vrl_exchange_elems(0, nullptr) != -1 || vrl_chunk_offset(nullptr, 0) != -1) {
        std::printf("a NULL dims argument was not rejected\n");
        ++bad;
    }
    if (valid_calls < iters / 40) {
        std::printf("only %d in-contract calls generated\n", valid_calls);
        ++bad;
    }
    std::printf("%s: %d calls, %d accepted (%d in-contract by construction), %d launches planned\n",
                bad ? "FAILED" : "abi fuzz ok", iters, accepted, valid_calls, g_launches);
    return bad ? 1 : 0;
}
