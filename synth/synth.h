/*
 * synth.h -- seeded synthetic gradients, shared by the test suite, the smoke
 * check and the benchmark on both sides of every parity comparison.
 *
 * It holds none of the all-reduce's arithmetic: only a counter-based random
 * source and its mapping to input values.  The same definitions are written
 * twice -- synth.c for the host, synth_fill.hip for the GPU -- with integer
 * arithmetic and single IEEE operations only, so both produce the same bits.
 *
 * Random source: SplitMix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; constants as published by
 * Vigna).  mix64(z) is its output function; a generator seeded with s returns
 * mix64(s + i*G) as output i = 1, 2, ... with G = 0x9E3779B97F4A7C15.
 *
 *   key(seed, rank)     = mix64(seed + (rank + 1) * G)
 *   word(seed, rank, i) = mix64(key(seed, rank) + (i + 1) * G)
 *
 * Value of element e of rank r:
 *   SYNTH_UNIFORM   u = word(e) >> 40 (24 bits); value = (u - 2^23) * 2^-23,
 *                   uniform on [-1, 1), exact in binary32
 *   SYNTH_NORMAL    Irwin-Hall approximation of N(0, sigma^2): the twelve
 *                   32-bit halves h of word(6e) .. word(6e+5) give the integer
 *                   T = 2*sum(h) - 12*(2^32 - 1), mean 0, var ~ 2^66;
 *                   value = f32(f64(T) * (sigma * 2^-33))
 *   SYNTH_RANKCONST value = rank + 1 (closed-form test)
 *   SYNTH_SMALLINT  value = (word(e) >> 57) - 64, an integer in [-64, 63]
 * For binary16 storage the binary32 value is rounded to nearest even.
 */
#ifndef SYNTH_H
#define SYNTH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { SYNTH_F32 = 0, SYNTH_F16 = 1 };
enum { SYNTH_UNIFORM = 0, SYNTH_NORMAL = 1, SYNTH_RANKCONST = 2, SYNTH_SMALLINT = 3 };

uint64_t synth_mix64(uint64_t z);
uint64_t synth_word(uint64_t seed, int rank, uint64_t i);

/* Elements [first, first + count) of rank `rank`, written to dst[0..count). */
void synth_fill_host(void *dst, int dtype, int dist, uint64_t seed, int rank,
                     uint64_t first, uint64_t count, double sigma);

/* Elements idx[0..count) of rank `rank`, written to dst[0..count). */
void synth_gather_host(void *dst, int dtype, int dist, uint64_t seed, int rank,
                       const uint64_t *idx, uint64_t count, double sigma);

/* binary32 -> binary16, round to nearest even (exported for its test) */
uint16_t synth_f32_to_f16(float x);

#ifdef __cplusplus
}
#endif
#endif
