// C ABI of libvrl.so: argument validation, launch planning, kernel launch.
//
// Every check runs before anything is enqueued, in this order: dimensions and
// window (VRL_E_INVALID), pointers and layouts (VRL_E_INVALID / VRL_E_LAYOUT),
// the launch plan's size limits (VRL_E_INVALID, vrl_plan.cpp), then the device, the
// stream's device and the pointers' allocations (VRL_E_DEVICE / VRL_E_INVALID).  All but the last
// group need no GPU, so they are exercised by the host-only tests.  The fail-closed behaviour (no silent fallback; layouts
// outside the contract are reported so the caller keeps its materialising
// path) follows the Vflash "Sol-Engine alignment" page, "What is enabled",
// and its note on incompatible layouts raising rather than falling back.
#include "../../include/vrl.h"
#include "vrl_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

// Only the C ABI is visible outside the library (built with -fvisibility=hidden).
#define VRL_EXPORT __attribute__((visibility("default")))

namespace {

thread_local char g_error[512];

vrl_status fail(vrl_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return s;
}

constexpr int64_t kMaxElems = int64_t(1) << 52;

// Dimensions and window.
vrl_status check_dims(const vrl_dims *d)
{
    if (!d)
        return fail(VRL_E_INVALID, "dims is NULL");
    if (d->P < 1 || d->C < 1 || d->s_local < 1 || d->H < 1 || d->D < 1)
        return fail(VRL_E_INVALID, "P, C, s_local, H and D must be >= 1 (P=%d C=%d s_local=%lld H=%d D=%d)",
                    d->P, d->C, (long long)d->s_local, d->H, d->D);
    if (d->H % d->P != 0)
        return fail(VRL_E_INVALID, "H=%d is not divisible by P=%d", d->H, d->P);
    if (d->chunk_heads != 0 && d->chunk_heads != 1)
        return fail(VRL_E_INVALID, "chunk_heads must be 0 or 1, got %d", d->chunk_heads);
    if (!d->chunk_heads && d->C > d->s_local)
        return fail(VRL_E_INVALID, "C=%d exceeds s_local=%lld (empty chunks)", d->C,
                    (long long)d->s_local);
    if (d->chunk_heads && (d->H / d->P) % d->C != 0)
        return fail(VRL_E_INVALID, "head group G=%d is not divisible by C=%d", d->H / d->P, d->C);
    const int64_t hd = int64_t(d->H) * d->D;
    if (d->s_local > kMaxElems / 3 / hd / d->P)
        return fail(VRL_E_INVALID, "problem too large");
    return VRL_OK;
}

vrl_status check_window(const vrl_dims *d, int32_t cb, int32_t ce)
{
    if (cb < 0 || ce > d->C || cb >= ce)
        return fail(VRL_E_INVALID, "bad chunk window [%d, %d) for C=%d", cb, ce, d->C);
    return VRL_OK;
}

// Geometry of a [rows][heads][D] view: its elements are
// ptr + 2 * (t * st + h * sh + e) bytes.  Strides of size-1 axes are
// irrelevant and taken as 0.
struct Geom {
    uintptr_t ptr;
    int64_t rows, heads, D, st, sh;
    bool output;
    const char *name;
};

Geom geom(const vrl_view *v, int64_t rows, int64_t heads, int64_t D, bool output, const char *name)
{
    Geom g{reinterpret_cast<uintptr_t>(v->ptr), rows, heads, D, v->stride_tok, v->stride_head,
           output, name};
    if (rows == 1)
        g.st = 0;
    if (heads == 1)
        g.sh = 0;
    return g;
}

Geom dense(const void *p, int64_t elems, bool output, const char *name)
{
    return Geom{reinterpret_cast<uintptr_t>(p), 1, 1, elems, 0, 0, output, name};
}

// Byte range [lo, hi) that holds every element of the view.
void span(const Geom &g, uintptr_t &lo, uintptr_t &hi)
{
    lo = g.ptr;
    hi = g.ptr + 2 * uintptr_t((g.rows - 1) * g.st + (g.heads - 1) * g.sh + g.D);
}

// True when no two elements of the view share an address: with the axes
// sorted by stride, each stride exceeds the reach of the faster axes.
bool self_disjoint(const Geom &g)
{
    struct Ax {
        int64_t n, s;
    } ax[3] = {{g.D, 1}, {g.heads, g.sh}, {g.rows, g.st}};
    std::sort(ax, ax + 3, [](const Ax &x, const Ax &y) { return x.s < y.s; });
    int64_t reach = 0;  // largest offset reachable with the faster axes
    for (const Ax &a : ax) {
        if (a.n == 1)
            continue;
        if (a.s <= reach)
            return false;
        reach += (a.n - 1) * a.s;
    }
    return true;
}

// Outer axis (larger stride) and the width of what the inner axes cover.
void outer_inner(const Geom &g, int64_t &outer_n, int64_t &outer_s, int64_t &width)
{
    if (g.st >= g.sh) {
        outer_n = g.rows, outer_s = g.st;
        width = (g.heads - 1) * g.sh + g.D;
    } else {
        outer_n = g.heads, outer_s = g.sh;
        width = (g.rows - 1) * g.st + g.D;
    }
}

// Conservative test that two views share no element: disjoint byte ranges,
// or the same strides with the second view's outer slices falling into the
// gaps between the first one's (e.g. Q/K/V column views of one fused row).
bool disjoint(const Geom &a, const Geom &b)
{
    uintptr_t alo, ahi, blo, bhi;
    span(a, alo, ahi);
    span(b, blo, bhi);
    if (ahi <= blo || bhi <= alo)
        return true;
    if (a.rows != b.rows || a.heads != b.heads || a.D != b.D || a.st != b.st || a.sh != b.sh)
        return false;
    int64_t n, s, w;
    outer_inner(a, n, s, w);
    if (n < 2 || s <= 0)
        return false;
    // m = (b - a) / 2 mod s, the offset of b's slices within a's period,
    // from the exact unsigned distance between the pointers.
    const bool ahead = b.ptr >= a.ptr;
    const uintptr_t dist = ahead ? b.ptr - a.ptr : a.ptr - b.ptr;
    if (dist % 2 != 0)
        return false;
    const int64_t rem = int64_t((dist / 2) % uintptr_t(s));
    const int64_t m = ahead || rem == 0 ? rem : s - rem;
    return m >= w && s - m >= w;
}

// Largest element offset any view may reach from its base; keeps every span
// and address computation far from 64-bit overflow.
constexpr int64_t kMaxReach = int64_t(1) << 48;

vrl_status check_layout(const Geom *gs, int n)
{
    for (int i = 0; i < n; ++i) {
        const Geom &g = gs[i];
        if (g.ptr == 0)
            return fail(VRL_E_INVALID, "%s is NULL", g.name);
        if (g.st < 0 || g.sh < 0)
            return fail(VRL_E_LAYOUT, "%s has a negative stride", g.name);
        if ((g.rows > 1 && g.st > kMaxReach / (g.rows - 1)) ||
            (g.heads > 1 && g.sh > kMaxReach / (g.heads - 1)) ||
            (g.rows - 1) * g.st + (g.heads - 1) * g.sh + g.D > kMaxReach)
            return fail(VRL_E_INVALID, "%s reaches beyond 2^48 elements", g.name);
        uintptr_t lo, hi;
        span(g, lo, hi);
        if (hi < lo)
            return fail(VRL_E_INVALID, "%s extends past the end of the address space", g.name);
        if (g.ptr % 2 != 0)
            return fail(VRL_E_LAYOUT, "%s is not 2-byte aligned", g.name);
        if (g.output && !self_disjoint(g))
            return fail(VRL_E_LAYOUT, "elements of output %s overlap each other", g.name);
    }
    // Inputs may share memory (e.g. Q/K/V views of one fused row); an output
    // may share none with any other argument.
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j)
            if ((gs[i].output || gs[j].output) && !disjoint(gs[i], gs[j]))
                return fail(VRL_E_LAYOUT, "%s overlaps %s", gs[i].name, gs[j].name);
    return VRL_OK;
}

// ---- device checks -----------------------------------------------------------

std::atomic<int> g_arch_ok[256];  // 0 unknown, 1 gfx950, 2 other

vrl_status check_device(int &dev)
{
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(VRL_E_DEVICE, "no current HIP device");
    }
    if (dev < 0 || dev >= 256)
        return fail(VRL_E_DEVICE, "device ordinal %d out of range", dev);
    int st = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(VRL_E_DEVICE, "cannot query device %d", dev);
        }
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_ok[dev].store(st, std::memory_order_relaxed);
    }
    if (st != 1)
        return fail(VRL_E_DEVICE, "device %d is not gfx950", dev);
    return VRL_OK;
}

// A stream other than the null stream must belong to `dev`: the memory
// checks below are made against that device, and a kernel enqueued on
// another device's stream would run there.
vrl_status check_stream(void *stream, int dev)
{
    if (!stream)
        return VRL_OK;
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(VRL_E_DEVICE, "cannot query the device of hip_stream");
    }
    if (sdev != dev)
        return fail(VRL_E_DEVICE, "hip_stream belongs to device %d, not the current device %d", int(sdev), dev);
    return VRL_OK;
}

// Each view must be device memory of `dev` and lie inside its allocation.
vrl_status check_memory(const Geom *gs, int n, int dev)
{
    for (int i = 0; i < n; ++i) {
        const Geom &g = gs[i];
        hipPointerAttribute_t attr;
        if (hipPointerGetAttributes(&attr, reinterpret_cast<void *>(g.ptr)) != hipSuccess) {
            (void)hipGetLastError();
            return fail(VRL_E_DEVICE, "%s is not HIP device memory", g.name);
        }
        if (attr.type != hipMemoryTypeDevice || attr.device != dev)
            return fail(VRL_E_DEVICE, "%s is not device memory of device %d", g.name, dev);
        hipDeviceptr_t base = nullptr;
        size_t size = 0;
        if (hipMemGetAddressRange(&base, &size, reinterpret_cast<hipDeviceptr_t>(g.ptr)) !=
            hipSuccess) {
            (void)hipGetLastError();
            return fail(VRL_E_DEVICE, "cannot find the allocation of %s", g.name);
        }
        uintptr_t lo, hi;
        span(g, lo, hi);
        const uintptr_t b = reinterpret_cast<uintptr_t>(base);
        if (lo < b || hi > b + size)
            return fail(VRL_E_INVALID, "%s extends past its allocation (%zu bytes)", g.name, size);
    }
    return VRL_OK;
}

vrl_status run(vrl::Op op, const vrl_dims *d, const Geom *views, int nviews, const Geom &wire,
               int32_t cb, int32_t ce, void *stream)
{
    Geom all[4];
    for (int i = 0; i < nviews; ++i)
        all[i] = views[i];
    all[nviews] = wire;
    vrl_status s = check_layout(all, nviews + 1);
    if (s != VRL_OK)
        return s;
    vrl::PlanView pv[3];
    for (int i = 0; i < nviews; ++i)
        pv[i] = vrl::PlanView{views[i].ptr, views[i].st, views[i].sh};
    const vrl::Problem pb{d->P, d->C, d->s_local, d->H, d->D, d->chunk_heads};
    vrl::LaunchPlan pl;
    const char *why = nullptr;
    if (!vrl::plan_launch(op, pb, pv, nviews, wire.ptr, cb, ce, pl, &why))
        return fail(VRL_E_INVALID, "%s", why);
    int dev = 0;
    if ((s = check_device(dev)) != VRL_OK)
        return s;
    if ((s = check_stream(stream, dev)) != VRL_OK)
        return s;
    if ((s = check_memory(all, nviews + 1, dev)) != VRL_OK)
        return s;
    const hipError_t e = vrl::launch(pl, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(VRL_E_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return VRL_OK;
}

bool null_view(const vrl_view *v)
{
    return v == nullptr;
}

}  // namespace

extern "C" {

VRL_EXPORT int64_t vrl_exchange_elems(int which, const vrl_dims *dims)
{
    g_error[0] = 0;
    if (check_dims(dims) != VRL_OK)
        return -1;
    if (which != VRL_EXCHANGE_QKV && which != VRL_EXCHANGE_ATTN) {
        fail(VRL_E_INVALID, "which must be VRL_EXCHANGE_QKV or VRL_EXCHANGE_ATTN, got %d", which);
        return -1;
    }
    return (which == VRL_EXCHANGE_QKV ? 3 : 1) * dims->s_local * dims->H * dims->D;
}

VRL_EXPORT int64_t vrl_chunk_offset(const vrl_dims *dims, int32_t c)
{
    g_error[0] = 0;
    if (check_dims(dims) != VRL_OK)
        return -1;
    if (c < 0 || c > dims->C) {
        fail(VRL_E_INVALID, "chunk index %d outside [0, C=%d]", c, dims->C);
        return -1;
    }
    if (dims->chunk_heads)
        return int64_t(c) * (dims->H / dims->P / dims->C);
    const int64_t q = dims->s_local / dims->C, r = dims->s_local % dims->C;
    return int64_t(c) * q + std::min<int64_t>(c, r);
}

VRL_EXPORT vrl_status vrl_qkv_pack(const vrl_dims *dims, const vrl_view *q, const vrl_view *k,
                        const vrl_view *v, void *packed, int32_t c_begin, int32_t c_end,
                        void *hip_stream)
{
    g_error[0] = 0;
    try {
        vrl_status s = check_dims(dims);
        if (s == VRL_OK)
            s = check_window(dims, c_begin, c_end);
        if (s != VRL_OK)
            return s;
        if (null_view(q) || null_view(k) || null_view(v))
            return fail(VRL_E_INVALID, "a view argument is NULL");
        const int64_t S_l = dims->s_local, H = dims->H, D = dims->D;
        const Geom views[3] = {geom(q, S_l, H, D, false, "q"), geom(k, S_l, H, D, false, "k"),
                               geom(v, S_l, H, D, false, "v")};
        const Geom wire = dense(packed, vrl_exchange_elems(VRL_EXCHANGE_QKV, dims), true, "packed");
        return run(vrl::Op::Pack, dims, views, 3, wire, c_begin, c_end, hip_stream);
    } catch (...) {
        return fail(VRL_E_DEVICE, "internal error");
    }
}

VRL_EXPORT vrl_status vrl_qkv_unpack(const vrl_dims *dims, const void *recv, const vrl_view *q,
                          const vrl_view *k, const vrl_view *v, int32_t c_begin, int32_t c_end,
                          void *hip_stream)
{
    g_error[0] = 0;
    try {
        vrl_status s = check_dims(dims);
        if (s == VRL_OK)
            s = check_window(dims, c_begin, c_end);
        if (s != VRL_OK)
            return s;
        if (null_view(q) || null_view(k) || null_view(v))
            return fail(VRL_E_INVALID, "a view argument is NULL");
        const int64_t S = int64_t(dims->P) * dims->s_local, G = dims->H / dims->P, D = dims->D;
        const Geom views[3] = {geom(q, S, G, D, true, "q"), geom(k, S, G, D, true, "k"),
                               geom(v, S, G, D, true, "v")};
        const Geom wire = dense(recv, vrl_exchange_elems(VRL_EXCHANGE_QKV, dims), false, "recv");
        return run(vrl::Op::Unpack, dims, views, 3, wire, c_begin, c_end, hip_stream);
    } catch (...) {
        return fail(VRL_E_DEVICE, "internal error");
    }
}

VRL_EXPORT vrl_status vrl_attn_split(const vrl_dims *dims, const vrl_view *o, void *send, int32_t c_begin,
                          int32_t c_end, void *hip_stream)
{
    g_error[0] = 0;
    try {
        vrl_status s = check_dims(dims);
        if (s == VRL_OK)
            s = check_window(dims, c_begin, c_end);
        if (s != VRL_OK)
            return s;
        if (null_view(o))
            return fail(VRL_E_INVALID, "view o is NULL");
        const int64_t S = int64_t(dims->P) * dims->s_local, G = dims->H / dims->P, D = dims->D;
        const Geom views[1] = {geom(o, S, G, D, false, "o")};
        const Geom wire = dense(send, vrl_exchange_elems(VRL_EXCHANGE_ATTN, dims), true, "send");
        return run(vrl::Op::Split, dims, views, 1, wire, c_begin, c_end, hip_stream);
    } catch (...) {
        return fail(VRL_E_DEVICE, "internal error");
    }
}

VRL_EXPORT vrl_status vrl_head_merge(const vrl_dims *dims, const void *recv, const vrl_view *out,
                          int32_t c_begin, int32_t c_end, void *hip_stream)
{
    g_error[0] = 0;
    try {
        vrl_status s = check_dims(dims);
        if (s == VRL_OK)
            s = check_window(dims, c_begin, c_end);
        if (s != VRL_OK)
            return s;
        if (null_view(out))
            return fail(VRL_E_INVALID, "view out is NULL");
        const int64_t S_l = dims->s_local, H = dims->H, D = dims->D;
        const Geom views[1] = {geom(out, S_l, H, D, true, "out")};
        const Geom wire = dense(recv, vrl_exchange_elems(VRL_EXCHANGE_ATTN, dims), false, "recv");
        return run(vrl::Op::Merge, dims, views, 1, wire, c_begin, c_end, hip_stream);
    } catch (...) {
        return fail(VRL_E_DEVICE, "internal error");
    }
}

VRL_EXPORT const char *vrl_status_string(vrl_status status)
{
    switch (status) {
    case VRL_OK: return "VRL_OK";
    case VRL_E_INVALID: return "VRL_E_INVALID";
    case VRL_E_LAYOUT: return "VRL_E_LAYOUT";
    case VRL_E_DEVICE: return "VRL_E_DEVICE";
    }
    return "VRL_E_UNKNOWN";
}

VRL_EXPORT const char *vrl_last_error(void)
{
    return g_error;
}

}  // extern "C"
