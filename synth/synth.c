/*
 * synth.c -- host side of the seeded synthetic gradients (definitions in
 * synth.h).  Multithreaded over elements with OpenMP when built with it; the
 * values do not depend on the thread count.
 */
#include "synth.h"

#include <string.h>

#define SYNTH_G 0x9E3779B97F4A7C15ull

uint64_t synth_mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static uint64_t key_of(uint64_t seed, int rank)
{
    return synth_mix64(seed + (uint64_t)(rank + 1) * SYNTH_G);
}

uint64_t synth_word(uint64_t seed, int rank, uint64_t i)
{
    return synth_mix64(key_of(seed, rank) + (i + 1) * SYNTH_G);
}

/* Round-to-nearest-even binary32 -> binary16 on the bit patterns. */
uint16_t synth_f32_to_f16(float x)
{
    uint32_t b;
    memcpy(&b, &x, 4);
    uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
    uint32_t e = (b >> 23) & 0xffu;
    uint32_t m = b & 0x7fffffu;
    if (e == 0xff) /* inf / nan */
        return sign | 0x7c00u | (m ? 0x200u : 0u);
    int E = (int)e - 127 + 15;   /* biased binary16 exponent */
    if (E >= 31)
        return sign | 0x7c00u;
    uint32_t mant;               /* significand incl. hidden bit, 24 bits */
    int shift;                   /* how many low bits are dropped */
    if (e == 0)
        return sign;             /* binary32 subnormals are < 2^-126: round to 0 */
    mant = m | 0x800000u;
    if (E >= 1)
        shift = 13;
    else
        shift = 14 - E;          /* result subnormal: value = mant * 2^(e-150) */
    if (shift > 25)
        return sign;             /* below half the smallest subnormal */
    uint32_t kept = mant >> shift;
    uint32_t rem = mant & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (kept & 1u)))
        kept += 1u;
    if (E >= 1) {
        /* kept in [2^10, 2^11]; carry into the exponent is handled by the add */
        uint32_t bits = ((uint32_t)E << 10) + (kept - 0x400u);
        if (bits >= 0x7c00u)
            return sign | 0x7c00u;
        return sign | (uint16_t)bits;
    }
    return sign | (uint16_t)kept; /* subnormal, or 0x400 = smallest normal */
}

static float value_f32(int dist, uint64_t seed, int rank, uint64_t e, double scale)
{
    switch (dist) {
    case SYNTH_UNIFORM: {
        int32_t u = (int32_t)(synth_word(seed, rank, e) >> 40);
        return (float)(u - (1 << 23)) * 0x1p-23f;
    }
    case SYNTH_NORMAL: {
        uint64_t k = key_of(seed, rank);
        int64_t s = 0;
        for (int j = 0; j < 6; ++j) {
            uint64_t w = synth_mix64(k + (6 * e + (uint64_t)j + 1) * SYNTH_G);
            s += (int64_t)(w & 0xffffffffull) + (int64_t)(w >> 32);
        }
        int64_t T = 2 * s - 12 * (int64_t)0xffffffffll;
        return (float)((double)T * scale);
    }
    case SYNTH_RANKCONST:
        return (float)(rank + 1);
    case SYNTH_SMALLINT:
    default:
        return (float)((int)(synth_word(seed, rank, e) >> 57) - 64);
    }
}

void synth_fill_host(void *dst, int dtype, int dist, uint64_t seed, int rank,
                     uint64_t first, uint64_t count, double sigma)
{
    double scale = sigma * 0x1p-33;
    long long n = (long long)count;
#pragma omp parallel for schedule(static)
    for (long long i = 0; i < n; ++i) {
        float v = value_f32(dist, seed, rank, first + (uint64_t)i, scale);
        if (dtype == SYNTH_F32)
            ((float *)dst)[i] = v;
        else
            ((uint16_t *)dst)[i] = synth_f32_to_f16(v);
    }
}

void synth_gather_host(void *dst, int dtype, int dist, uint64_t seed, int rank,
                       const uint64_t *idx, uint64_t count, double sigma)
{
    double scale = sigma * 0x1p-33;
    for (uint64_t i = 0; i < count; ++i) {
        float v = value_f32(dist, seed, rank, idx[i], scale);
        if (dtype == SYNTH_F32)
            ((float *)dst)[i] = v;
        else
            ((uint16_t *)dst)[i] = synth_f32_to_f16(v);
    }
}
