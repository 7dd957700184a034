// kernels.hip -- gfx950 kernels of the gradient all-reduce.
//
// All kernels are HBM-streaming: one 16-byte (dwordx4) access per lane per
// vector, 256-lane workgroups, one tile of a chunk per workgroup.  There is
// no contraction here, so no MFMA: an element of a step costs 3 (reduce) or
// 2 (gather) element transfers, an element of the fused pass 2P, against
// at most P-1 adds.
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
//    "总结": gradients are averaged).
#include <hip/hip_runtime.h>

#include "ddl_internal.h"

namespace ddl {
namespace {

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

struct F32 {
    using T = float;
    using V = f32x4;
    static constexpr int N = 4;
    __device__ static V add(V a, V b) { return a + b; }
    __device__ static V div(V a, float d) { return a / d; }
    __device__ static T add1(T a, T b) { return a + b; }
    __device__ static T div1(T a, float d) { return a / d; }
};

struct F16 {
    using T = _Float16;
    using V = f16x8;
    static constexpr int N = 8;
    __device__ static V add(V a, V b) {
        f32x8 s = __builtin_convertvector(a, f32x8) + __builtin_convertvector(b, f32x8);
        return __builtin_convertvector(s, f16x8);
    }
    __device__ static V div(V a, float d) {
        f32x8 q = opaque(__builtin_convertvector(a, f32x8) / d);
        return __builtin_convertvector(q, f16x8);
    }
    __device__ static T add1(T a, T b) { return (T)((float)a + (float)b); }
    __device__ static T div1(T a, float d) { return (T)opaque1((float)a / d); }
};

template <class V>
__device__ __forceinline__ V ldv(const void *p) {
    return *reinterpret_cast<const V *>(p);
}
template <class V>
__device__ __forceinline__ void stv(void *p, V v) {
    *reinterpret_cast<V *>(p) = v;
}

// Largest i in [lo, hi) with prefix[i] <= tile (prefix is non-decreasing,
// prefix[lo] <= tile < prefix[hi]).  Uniform across the workgroup.
__device__ __forceinline__ uint32_t find_item(const uint32_t *__restrict__ prefix,
                                              uint32_t lo, uint32_t hi, uint32_t tile) {
    while (hi - lo > 1) {
        uint32_t mid = lo + ((hi - lo) >> 1);
        if (prefix[mid] <= tile)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// step kernels: one launch = one schedule step over every pair of every ring
// of every bucket in the group.  Reduce: dst = dst (+) src (then / P when the
// item completes its chunk's sum).  Gather: dst = src.
// ---------------------------------------------------------------------------
template <class E, bool kReduce>
__global__ __launch_bounds__(kBlock) void step_kernel(RankPtrs bufs, StepArgs a) {
    using T = typename E::T;
    using V = typename E::V;
    constexpr uint64_t kTile = step_tile_elems(sizeof(T));
    const uint32_t tile = a.tile_base + blockIdx.x;
    const uint32_t i = find_item(a.prefix, a.item_lo, a.item_hi, tile);
    const DevItem it = a.items[i];
    const uint64_t t0 = (uint64_t)(tile - a.prefix[i]) * kTile;
    const uint64_t rem = it.len - t0;
    const uint32_t cnt = (uint32_t)(rem < kTile ? rem : kTile);
    T *dst = static_cast<T *>(bufs.p[it.dst]) + it.off + t0;
    const T *src = static_cast<const T *>(bufs.p[it.src]) + it.off + t0;
    const bool divide = kReduce && (it.flags & kItemDivide);
    const uint32_t tid = threadIdx.x;
    uint32_t done = 0;
    if (it.flags & kItemAligned) {
        const uint32_t nvec = cnt / E::N;
        if (nvec == (uint32_t)(kStepVecsPerLane * kBlock)) {
            V s[kStepVecsPerLane], d[kStepVecsPerLane];
#pragma unroll
            for (int j = 0; j < kStepVecsPerLane; ++j) {
                s[j] = ldv<V>(src + (size_t)(j * kBlock + tid) * E::N);
                if (kReduce)
                    d[j] = ldv<V>(dst + (size_t)(j * kBlock + tid) * E::N);
            }
#pragma unroll
            for (int j = 0; j < kStepVecsPerLane; ++j) {
                V r = s[j];
                if (kReduce) {
                    r = E::add(d[j], s[j]);
                    if (divide)
                        r = E::div(r, a.divisor);
                }
                stv<V>(dst + (size_t)(j * kBlock + tid) * E::N, r);
            }
        } else {
            for (uint32_t v = tid; v < nvec; v += kBlock) {
                V r = ldv<V>(src + (size_t)v * E::N);
                if (kReduce) {
                    r = E::add(ldv<V>(dst + (size_t)v * E::N), r);
                    if (divide)
                        r = E::div(r, a.divisor);
                }
                stv<V>(dst + (size_t)v * E::N, r);
            }
        }
        done = nvec * E::N;
    }
    // element-wise: the ragged end of a segment, or a whole item whose
    // offset is not vector aligned
    for (uint32_t e = done + tid; e < cnt; e += kBlock) {
        T r = src[e];
        if (kReduce) {
            r = E::add1(dst[e], r);
            if (divide)
                r = E::div1(r, a.divisor);
        }
        dst[e] = r;
    }
}

// ---------------------------------------------------------------------------
// fused pass: every element is read once from each of the P ranks, summed in
// the order the schedule sums it -- chain[0..P) in groups of `group`
// entries, each group left to right, then the group sums left to right --
// divided by P for the mean, and written once to each rank.
//
// The rank pointers, in chain order, are staged in LDS before the first
// store, so the data loads never wait behind a table load; they are issued
// eight at a time ahead of the serial add chain.
// ---------------------------------------------------------------------------
template <class E>
struct Chain {
    using V = typename E::V;
    V acc = {}, gacc = {};
    int pos = 0;
    bool first_group = true;
    __device__ __forceinline__ void push(V x, int group) {
        gacc = pos == 0 ? x : E::add(gacc, x);
        if (++pos == group) {
            acc = first_group ? gacc : E::add(acc, gacc);
            first_group = false;
            pos = 0;
        }
    }
};

// Sum of element vector e over the chain.  Ungrouped (rings): one chain of
// P entries.  Grouped (torus): chains of `group` entries, then their sums.
template <class E, bool kGrouped>
__device__ __forceinline__ typename E::V fused_vec(const typename E::T *const *sp, int P,
                                                   int group, uint64_t e) {
    using V = typename E::V;
    if (!kGrouped) {
        V acc = ldv<V>(sp[0] + e);
        int b = 1;
        for (; b + 8 <= P; b += 8) {
            V x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                x[j] = ldv<V>(sp[b + j] + e);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc = E::add(acc, x[j]);
        }
        for (; b < P; ++b)
            acc = E::add(acc, ldv<V>(sp[b] + e));
        return acc;
    }
    Chain<E> c;
    int b = 0;
    for (; b + 8 <= P; b += 8) {
        V x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = ldv<V>(sp[b + j] + e);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            c.push(x[j], group);
    }
    for (; b < P; ++b)
        c.push(ldv<V>(sp[b] + e), group);
    return c.acc;
}

template <class E, bool kGrouped>
__global__ __launch_bounds__(kBlock) void fused_kernel(RankPtrs bufs, FusedArgs a) {
    using T = typename E::T;
    using V = typename E::V;
    constexpr uint64_t kTile = fused_tile_elems(sizeof(T));
    __shared__ const T *src[DDL_MAX_RANKS];
    const uint32_t tile = a.tile_base + blockIdx.x;
    const uint32_t i = find_item(a.prefix, a.span_lo, a.span_hi, tile);
    const DevSpan sp = a.spans[i];
    const int P = a.P;
    const uint32_t tid = threadIdx.x;
    if (tid < (uint32_t)P)
        src[tid] = static_cast<const T *>(bufs.p[a.chains[sp.chain_off + tid]]);
    __syncthreads();
    const uint64_t t0 = (uint64_t)(tile - a.prefix[i]) * kTile;
    const uint64_t rem = sp.len - t0;
    const uint32_t cnt = (uint32_t)(rem < kTile ? rem : kTile);
    const uint64_t base = sp.off + t0;
    uint32_t done = 0;
    if (sp.flags & kItemAligned) {
        const uint32_t nvec = cnt / E::N;
        for (uint32_t v = tid; v < nvec; v += kBlock) {
            const uint64_t e = base + (uint64_t)v * E::N;
            V acc = fused_vec<E, kGrouped>(src, P, a.group, e);
            if (a.mean)
                acc = E::div(acc, a.divisor);
            for (int r = 0; r < P; ++r)
                stv<V>(static_cast<T *>(bufs.p[r]) + e, acc);
        }
        done = nvec * E::N;
    }
    for (uint32_t k = done + tid; k < cnt; k += kBlock) {
        const uint64_t e = base + k;
        T acc = 0, gacc = 0;
        int pos = 0;
        bool first_group = true;
        for (int j = 0; j < P; ++j) {
            T x = src[j][e];
            gacc = pos == 0 ? x : E::add1(gacc, x);
            if (++pos == a.group) {
                acc = first_group ? gacc : E::add1(acc, gacc);
                first_group = false;
                pos = 0;
            }
        }
        if (a.mean)
            acc = E::div1(acc, a.divisor);
        for (int r = 0; r < P; ++r)
            static_cast<T *>(bufs.p[r])[e] = acc;
    }
}

}  // namespace

int launch_step(int dtype, int kind, const RankPtrs &bufs, const StepArgs &a,
                uint32_t tiles, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    dim3 grid(tiles), block(kBlock);
    if (dtype == DDL_F32) {
        if (kind == DDL_K_REDUCE)
            hipLaunchKernelGGL((step_kernel<F32, true>), grid, block, 0, s, bufs, a);
        else
            hipLaunchKernelGGL((step_kernel<F32, false>), grid, block, 0, s, bufs, a);
    } else {
        if (kind == DDL_K_REDUCE)
            hipLaunchKernelGGL((step_kernel<F16, true>), grid, block, 0, s, bufs, a);
        else
            hipLaunchKernelGGL((step_kernel<F16, false>), grid, block, 0, s, bufs, a);
    }
    return (int)hipGetLastError();
}

int launch_fused(int dtype, const RankPtrs &bufs, const FusedArgs &a, uint32_t tiles,
                 void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    dim3 grid(tiles), block(kBlock);
    const bool grouped = a.group != a.P;
    if (dtype == DDL_F32) {
        if (grouped)
            hipLaunchKernelGGL((fused_kernel<F32, true>), grid, block, 0, s, bufs, a);
        else
            hipLaunchKernelGGL((fused_kernel<F32, false>), grid, block, 0, s, bufs, a);
    } else {
        if (grouped)
            hipLaunchKernelGGL((fused_kernel<F16, true>), grid, block, 0, s, bufs, a);
        else
            hipLaunchKernelGGL((fused_kernel<F16, false>), grid, block, 0, s, bufs, a);
    }
    return (int)hipGetLastError();
}

}  // namespace ddl
