// device_common.h -- element types, vector accesses and the tile lookup
// shared by the step kernels and the fused kernel (gfx950).
//
// Arithmetic follows the schedule exactly:
//  - binary32: a + b in round-to-nearest-even with subnormals kept (the
//    library is built without fast-math or denormal flushing, and with
//    packed fp32 math disabled);
//  - binary16 (Sony "224秒训练ResNet-50" article, "训练设置": FP16 gradient
//    exchange): every add is done in binary32 and rounded to binary16, the
//    type the partial sums travel in between steps;
//  - mean: one correctly rounded binary32 division by P (binary16: of the
//    value widened to binary32, then rounded to binary16), fused into the
//    store of the add that completes the sum (Baidu Ring-Allreduce article,
//    "总结": gradients are averaged).  Binary16 takes the cheaper
//    quotient_by_rank below, which rounds to the same binary16 value.
#pragma once

#include <hip/hip_runtime.h>

#include "ddl_internal.h"

namespace ddl {
namespace dev {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Keeps the compiler from narrowing "binary32 divide, then round to
// binary16" into a binary16 divide, whose lowering is not the correctly
// rounded binary32 quotient this library promises.
__device__ __forceinline__ f32x8 opaque(f32x8 v) {
    asm volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ float opaque1(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

// x / d rounded to binary16 as RN16(RN32(x / d)) does, for x a binary16
// value widened to binary32 and d a rank count in [1, 128], with r =
// RN32(1 / d): q = RN32(x r) is within 2^-23 of x / d (relative), and
// e = x - q d is exact (x and q d are multiples of ulp(q), |e| <= 1.5 d
// ulps), so c = RN32(q + e r) is x / d up to 2^-47 (relative).  x / d is
// either a binary16 midpoint -- then c equals it exactly and both round the
// tie the same way -- or at least 2^-18 (relative; 2^-32 absolute among the
// subnormals) away from every midpoint, so that c, q's error far smaller,
// rounds to the same binary16 value as x / d, and x / d as RN32(x / d).
// e = 0 (x exact in q, +-0 included: c would lose the sign of -0) and
// non-finite x (e is NaN) keep q.  Every binary16 x at every d is checked
// against numpy's binary32 division on the device.
__device__ __forceinline__ float quotient_by_rank(float x, float d, float r) {
    const float q = x * r;
    const float e = __builtin_fmaf(-q, d, x);
    const float c = __builtin_fmaf(e, r, q);
    return (e != 0.0f && e == e) ? c : q;
}

// E::W is the binary32 vector of the N elements of one E::V (the weights
// of the SGD step are binary32 whatever the gradient type).
struct F32 {
    using T = float;
    using V = f32x4;
    using W = f32x4;
    static constexpr int N = 4;
    __device__ static W widen(V a) { return a; }
    __device__ static V add(V a, V b) { return a + b; }
    __device__ static V div(V a, float d) { return a / d; }
    __device__ static T add1(T a, T b) { return a + b; }
    __device__ static T div1(T a, float d) { return a / d; }
};

struct F16 {
    using T = _Float16;
    using V = f16x8;
    using W = f32x8;
    static constexpr int N = 8;
    __device__ static W widen(V a) { return __builtin_convertvector(a, f32x8); }
    __device__ static V add(V a, V b) {
        f32x8 s = __builtin_convertvector(a, f32x8) + __builtin_convertvector(b, f32x8);
        return __builtin_convertvector(s, f16x8);
    }
    __device__ static V div(V a, float d) {
        const float r = 1.0f / d;
        f32x8 x = __builtin_convertvector(a, f32x8), q;
#pragma unroll
        for (int i = 0; i < N; ++i)
            q[i] = quotient_by_rank(x[i], d, r);
        return __builtin_convertvector(opaque(q), f16x8);
    }
    __device__ static T add1(T a, T b) { return (T)((float)a + (float)b); }
    __device__ static T div1(T a, float d) {
        return (T)opaque1(quotient_by_rank((float)a, d, 1.0f / d));
    }
};

// The SGD step w - lr * y in binary32: the product is rounded before the
// difference (the library is built with -ffp-contract=off, so no fused
// multiply-add is formed).
template <class W>
__device__ __forceinline__ W sgd_step(W w, W y, float lr) {
    const W step = y * lr;
    return w - step;
}

template <class V>
__device__ __forceinline__ V ldv(const void *p) {
    return *reinterpret_cast<const V *>(p);
}
template <class V>
__device__ __forceinline__ void stv(void *p, V v) {
    *reinterpret_cast<V *>(p) = v;
}
// Sum over the workgroup of one binary64 value per lane: a butterfly within
// each wave64, then the waves' sums in wave order.  The result is in lane 0
// of wave 0.  Every lane of the workgroup must call it (it holds a barrier).
__device__ __forceinline__ double block_sum(double v, double *lds) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    if (lane == 0)
        lds[wave] = v;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0)
        for (int i = 0; i < kBlock / 64; ++i)
            s += lds[i];
    return s;
}

// acc += the square of every binary32 component of x, in binary64 (each
// square of a binary32 value is exact there), components in order.
template <class W>
__device__ __forceinline__ void add_squares(W x, double &acc) {
#pragma unroll
    for (int i = 0; i < (int)(sizeof(W) / sizeof(float)); ++i)
        acc += (double)x[i] * (double)x[i];
}

// Largest i in [lo, hi) with prefix[i] <= tile (prefix is non-decreasing,
// prefix[lo] <= tile < prefix[hi]).  Uniform across the workgroup.
//
// The items of a step are near-equal chunks, so the first probe is the
// item a uniform spread of the tiles would give; it is checked with two
// independent loads and, when it misses (skewed tables: buckets of very
// different sizes in one group), bounds a binary search.  Two rounds of
// loads instead of log2(items) dependent ones: a step's workgroups are
// short-lived, and the search is on their critical path.
__device__ __forceinline__ uint32_t find_item(const uint32_t *__restrict__ prefix,
                                              uint32_t lo, uint32_t hi, uint32_t tile) {
    if (hi - lo > 1) {
        const uint32_t t0 = prefix[lo], t1 = prefix[hi];
        const uint32_t g =
            lo + (uint32_t)((uint64_t)(tile - t0) * (uint64_t)(hi - lo) / (uint64_t)(t1 - t0));
        const uint32_t a = prefix[g], b = prefix[g + 1];
        if (a <= tile && tile < b)
            return g;
        if (a > tile)
            hi = g;
        else
            lo = g + 1;
    }
    while (hi - lo > 1) {
        uint32_t mid = lo + ((hi - lo) >> 1);
        if (prefix[mid] <= tile)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

}  // namespace dev
}  // namespace ddl
