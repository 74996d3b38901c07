/*
 * Seeded synthetic BF16 input generator.
 *
 * Shared input source for the oracle and for the device path: it draws
 * values and nothing else (no layout, chunking or relayout arithmetic
 * lives here).  Every value is a pure function of (seed, stream, index),
 * so the output does not depend on the number of threads that fill it.
 *
 * Random bits: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  Its i-th output from
 * state z is mix(z + (i + 1) * GOLDEN), with the finalizer below, so it is
 * counter-based and can be evaluated at any index directly.
 *
 * Normal values: Box-Muller transform in double precision (Box and
 * Muller, 1958), rounded double -> float -> bfloat16 (round to nearest
 * even).  Uniform values: u * 16 - 8 on [-8, 8), with about one element in
 * 32 replaced by +0, -0 or a random signed subnormal so that bit-level
 * moves of those patterns are exercised.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t sm_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Starting state of one (seed, stream) sequence. */
static inline uint64_t sm_key(uint64_t seed, uint64_t stream)
{
    return sm_mix(seed + GOLDEN) ^ sm_mix(stream * 0xD1B54A32D192ED03ull + 0x8CB92BA72F3D8DD7ull);
}

/* i-th SplitMix64 output of the sequence that starts at state z. */
static inline uint64_t sm_at(uint64_t z, uint64_t i)
{
    return sm_mix(z + (i + 1) * GOLDEN);
}

static inline uint16_t f32_to_bf16_rne(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu))
        return (uint16_t)((b >> 16) | 0x40u); /* quiet NaN, keeps sign */
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

/* Fills out[0..n) with N(0,1) samples of sequence (seed, stream). */
void dg_normal_bf16(uint16_t *out, int64_t n, uint64_t seed, uint64_t stream)
{
    const uint64_t z = sm_key(seed, stream);
    const int64_t pairs = (n + 1) / 2;
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < pairs; ++j) {
        uint64_t a = sm_at(z, 2 * (uint64_t)j);
        uint64_t b = sm_at(z, 2 * (uint64_t)j + 1);
        double u1 = ((double)(a >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
        double u2 = (double)(b >> 11) * 0x1.0p-53;         /* [0, 1) */
        double rad = sqrt(-2.0 * log(u1));
        double th = two_pi * u2;
        out[2 * j] = f32_to_bf16_rne((float)(rad * cos(th)));
        if (2 * j + 1 < n)
            out[2 * j + 1] = f32_to_bf16_rne((float)(rad * sin(th)));
    }
}

/* Fills out[0..n) with U[-8, 8) samples plus injected +0 / -0 / subnormals. */
void dg_uniform8_bf16(uint16_t *out, int64_t n, uint64_t seed, uint64_t stream)
{
    const uint64_t zu = sm_key(seed, stream);
    const uint64_t zs = sm_key(seed ^ 0x5DEECE66Dull, stream + 0x100000000ull);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t r = sm_at(zu, (uint64_t)i);
        uint64_t s = sm_at(zs, (uint64_t)i);
        double u = (double)(r >> 11) * 0x1.0p-53;
        uint16_t v = f32_to_bf16_rne((float)(u * 16.0 - 8.0));
        if ((s & 31u) == 0) {
            uint32_t kind = (uint32_t)((s >> 5) % 3u);
            if (kind == 0)
                v = 0x0000u;
            else if (kind == 1)
                v = 0x8000u;
            else
                v = (uint16_t)((((s >> 7) & 1u) << 15) | (((s >> 8) & 0x7Fu) | 1u));
        }
        out[i] = v;
    }
}

/* Raw SplitMix64 outputs, exposed so tests can check the generator against
 * the published reference values of SplitMix64. */
void dg_splitmix64(uint64_t *out, int64_t n, uint64_t state)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = sm_at(state, (uint64_t)i);
}
