// The C ABI used from C++ alone (no Python, no torch): hipMalloc'd buffers,
// a stream of its own, and the whole relayout path for P ranks in one GPU --
// pack, exchange (block copies), unpack, split of one plane, exchange, merge
// -- which must return that plane of every rank's input bit for bit.  Also
// checks a few error statuses and the host helpers.  Prints one line and
// exits 0 on success.
#include "../../include/vrl.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#define HIP_OK(x)                                                                       \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(2);                                                               \
        }                                                                               \
    } while (0)

#define VRL_OK_(x)                                                                        \
    do {                                                                                  \
        vrl_status s_ = (x);                                                              \
        if (s_ != VRL_OK) {                                                               \
            std::printf("%s at line %d: %s\n", vrl_status_string(s_), __LINE__, vrl_last_error()); \
            std::exit(3);                                                                 \
        }                                                                                 \
    } while (0)

struct Case {
    int32_t P, C;
    int64_t S_l;
    int32_t H, D, chunk_heads;
    bool head_major;  // attention-side Q/K/V stored [G][S][D]
};

static uint64_t rng_state = 0x243F6A8885A308D3ull;
static uint16_t next16()
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return uint16_t(rng_state >> 17);
}

static bool run(const Case &k, hipStream_t st)
{
    const vrl_dims d{k.P, k.C, k.S_l, k.H, k.D, k.chunk_heads};
    const int64_t G = k.H / k.P, S = k.P * k.S_l, HD = int64_t(k.H) * k.D;
    const int64_t n_qkv = vrl_exchange_elems(VRL_EXCHANGE_QKV, &d);
    const int64_t n_att = vrl_exchange_elems(VRL_EXCHANGE_ATTN, &d);
    if (n_qkv != 3 * k.S_l * HD || n_att != k.S_l * HD)
        return false;
    const int plane = 1;

    std::vector<std::vector<uint16_t>> host(k.P, std::vector<uint16_t>(k.S_l * 3 * HD));
    std::vector<uint16_t *> fused(k.P), packed(k.P), recv(k.P), send(k.P), back(k.P), merged(k.P);
    std::vector<uint16_t *> planes(3 * k.P);
    for (int r = 0; r < k.P; ++r) {
        for (auto &x : host[r])
            x = next16();
        HIP_OK(hipMalloc(&fused[r], host[r].size() * 2));
        HIP_OK(hipMemcpy(fused[r], host[r].data(), host[r].size() * 2, hipMemcpyHostToDevice));
        HIP_OK(hipMalloc(&packed[r], n_qkv * 2));
        HIP_OK(hipMalloc(&recv[r], n_qkv * 2));
        HIP_OK(hipMalloc(&send[r], n_att * 2));
        HIP_OK(hipMalloc(&back[r], n_att * 2));
        HIP_OK(hipMalloc(&merged[r], n_att * 2));
        for (int q = 0; q < 3; ++q)
            HIP_OK(hipMalloc(&planes[3 * r + q], S * G * k.D * 2));
    }
    // the attention side: token-major [S][G][D] or head-major [G][S][D]
    const int64_t a_st = k.head_major ? k.D : G * k.D;
    const int64_t a_sh = k.head_major ? S * k.D : k.D;

    for (int r = 0; r < k.P; ++r) {
        vrl_view q{fused[r], 3 * HD, k.D}, kk{fused[r] + HD, 3 * HD, k.D}, v{fused[r] + 2 * HD, 3 * HD, k.D};
        VRL_OK_(vrl_qkv_pack(&d, &q, &kk, &v, packed[r], 0, k.C, st));
    }
    // exchange: the part of sender s for peer r -> the part of r from s
    for (int s = 0; s < k.P; ++s)
        for (int r = 0; r < k.P; ++r)
            HIP_OK(hipMemcpyAsync(recv[r] + s * (n_qkv / k.P), packed[s] + r * (n_qkv / k.P),
                                  n_qkv / k.P * 2, hipMemcpyDeviceToDevice, st));
    for (int r = 0; r < k.P; ++r) {
        vrl_view o[3];
        for (int q = 0; q < 3; ++q)
            o[q] = vrl_view{planes[3 * r + q], a_st, a_sh};
        VRL_OK_(vrl_qkv_unpack(&d, recv[r], &o[0], &o[1], &o[2], 0, k.C, st));
        VRL_OK_(vrl_attn_split(&d, &o[plane], send[r], 0, k.C, st));
    }
    for (int s = 0; s < k.P; ++s)
        for (int r = 0; r < k.P; ++r)
            HIP_OK(hipMemcpyAsync(back[r] + s * (n_att / k.P), send[s] + r * (n_att / k.P),
                                  n_att / k.P * 2, hipMemcpyDeviceToDevice, st));
    for (int r = 0; r < k.P; ++r) {
        vrl_view out{merged[r], HD, k.D};
        VRL_OK_(vrl_head_merge(&d, back[r], &out, 0, k.C, st));
    }
    HIP_OK(hipStreamSynchronize(st));

    bool ok = true;
    std::vector<uint16_t> got(n_att);
    for (int r = 0; r < k.P && ok; ++r) {
        HIP_OK(hipMemcpy(got.data(), merged[r], n_att * 2, hipMemcpyDeviceToHost));
        for (int64_t t = 0; t < k.S_l && ok; ++t)
            ok = std::memcmp(&got[t * HD], &host[r][t * 3 * HD + plane * HD], HD * 2) == 0;
    }
    for (int r = 0; r < k.P; ++r) {
        HIP_OK(hipFree(fused[r]));
        HIP_OK(hipFree(packed[r]));
        HIP_OK(hipFree(recv[r]));
        HIP_OK(hipFree(send[r]));
        HIP_OK(hipFree(back[r]));
        HIP_OK(hipFree(merged[r]));
        for (int q = 0; q < 3; ++q)
            HIP_OK(hipFree(planes[3 * r + q]));
    }
    return ok;
}

int main()
{
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    const Case cases[] = {
        {2, 4, 27707, 56, 128, 0, false},  // the representative shape
        {2, 4, 27707, 56, 128, 1, false},  // same, chunks over heads
        {4, 4, 7752, 32, 128, 0, true},    // P = 4, head-major attention side
        {3, 5, 101, 12, 64, 0, false},     // ragged chunks
        {8, 2, 33, 16, 24, 1, true},
        {1, 1, 1, 1, 2, 0, false},         // the smallest problem
    };
    for (const Case &k : cases) {
        if (!run(k, st)) {
            std::printf("round trip FAILED: P=%d C=%d S_l=%lld H=%d D=%d chunk_heads=%d head_major=%d\n",
                        k.P, k.C, (long long)k.S_l, k.H, k.D, k.chunk_heads, int(k.head_major));
            return 1;
        }
    }
    // error statuses: nothing launched, a reason recorded
    const vrl_dims bad{3, 1, 8, 8, 8, 0};
    vrl_view v0{nullptr, 0, 0};
    if (vrl_qkv_pack(&bad, &v0, &v0, &v0, nullptr, 0, 1, st) != VRL_E_INVALID || !vrl_last_error()[0])
        return 1;
    const vrl_dims d{2, 4, 16, 8, 8, 0};
    if (vrl_chunk_offset(&d, 4) != 16 || vrl_chunk_offset(&d, 5) != -1)
        return 1;
    HIP_OK(hipStreamDestroy(st));
    std::printf("C ABI round trip ok (%zu cases)\n", sizeof(cases) / sizeof(cases[0]));
    return 0;
}
