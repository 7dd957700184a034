// step_kernels.hip -- one launch per schedule step (gfx950).
//
// A launch covers every pair of every ring of every bucket in the group: the
// schedule is race-free within a step, so all pairs run at once.  Each lane
// moves dwordx4 vectors of one source and one destination chunk.  The
// stores stay cached: the next step reads what this one wrote.
#include <type_traits>

#include "device_common.h"

// global (address space 1) accesses from addresses kept in LDS
#define DDL_STEP_GLOBAL __attribute__((address_space(1)))

namespace ddl {
namespace {

using namespace dev;

// ---------------------------------------------------------------------------
// step kernels: one launch = one schedule step over every pair of every ring
// of every bucket in the group.  Reduce: dst = dst (+) src (then / P when the
// item completes its chunk's sum).  Gather: dst = src.
//
// With kSgd the weights take their SGD step where the reduced value reaches
// a rank: the owner at the add that completes the sum (kItemFinal), every
// other rank when the all-gather delivers it (one replica per rank), or the
// owner alone (one shared replica).
// ---------------------------------------------------------------------------
template <class E, bool kReduce, bool kSgd, int VPL>
__device__ __forceinline__ void step_body(const RankPtrs &bufs, const StepArgs &a,
                                          const SgdArgs *g) {
    using T = typename E::T;
    using V = typename E::V;
    using W = typename E::W;
    constexpr uint64_t kTile = step_tile_elems(sizeof(T), VPL);
    const uint32_t tile = a.tile_base + blockIdx.x;
    const uint32_t i = find_item(a.prefix, a.item_lo, a.item_hi, tile);
    const DevItem it = a.items[i];
    const uint64_t j = tile - a.prefix[i];
    const uint64_t sh = tile_shift(it.off, kTile, a.anchor);
    const uint64_t lo = tile_lo(it.off, sh, kTile, j);
    const uint32_t cnt = (uint32_t)(tile_hi(it.off, it.len, sh, kTile, j) - lo);
    T *dst = static_cast<T *>(bufs.p[it.dst]) + lo;
    const T *src = static_cast<const T *>(bufs.p[it.src]) + lo;
    const bool divide = kReduce && (it.flags & kItemDivide);
    float *w = nullptr;
    float lr = 0.0f;
    if (kSgd && (kReduce ? (it.flags & kItemFinal) != 0 : g->nweights > 1)) {
        w = static_cast<float *>(g->w.p[g->nweights == 1 ? 0 : it.dst]) + lo;
        lr = g->lr;
    }
    const uint32_t tid = threadIdx.x;
    uint32_t done = 0;
    if (it.flags & kItemAligned) {
        const uint32_t nvec = cnt / E::N;
        if (nvec == (uint32_t)(VPL * kBlock)) {
            V s[VPL], d[VPL];
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                s[j] = ldv<V>(src + (size_t)(j * kBlock + tid) * E::N);
                if (kReduce)
                    d[j] = ldv<V>(dst + (size_t)(j * kBlock + tid) * E::N);
            }
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                V r = s[j];
                if (kReduce) {
                    r = E::add(d[j], s[j]);
                    if (divide)
                        r = E::div(r, a.divisor);
                }
                stv<V>(dst + (size_t)(j * kBlock + tid) * E::N, r);
                if (kSgd && w) {
                    float *wp = w + (size_t)(j * kBlock + tid) * E::N;
                    stv<W>(wp, sgd_step<W>(ldv<W>(wp), E::widen(r), lr));
                }
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
                if (kSgd && w) {
                    float *wp = w + (size_t)v * E::N;
                    stv<W>(wp, sgd_step<W>(ldv<W>(wp), E::widen(r), lr));
                }
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
        if (kSgd && w)
            w[e] = sgd_step<float>(w[e], (float)r, lr);
    }
}

template <class E, bool kReduce, int VPL>
__global__ __launch_bounds__(kBlock) void step_kernel(RankPtrs bufs, StepArgs a) {
    step_body<E, kReduce, false, VPL>(bufs, a, nullptr);
}

template <class E, bool kReduce, int VPL>
__global__ __launch_bounds__(kBlock) void step_sgd_kernel(RankPtrs bufs, StepArgs a,
                                                          SgdArgs g) {
    step_body<E, kReduce, true, VPL>(bufs, a, &g);
}

// ---------------------------------------------------------------------------
// persistent step kernel: one launch walks every schedule step of a group.
//
// Every dependency of the schedule is per element: the value that step t
// writes to element e of a rank is read again only at element e, by a later
// step.  So a workgroup that owns one tile of a fused span (a chunk, or a
// torus sub-piece, whose elements all follow the same chain of ranks) can
// run every step of the schedule over that tile by itself, in step order,
// and each lane touches the same elements at every step -- it reads back
// only what it wrote itself, so no barrier and no grid-wide wait is needed.
// Each step still moves its data through memory exactly as the one-launch-
// per-step path does (reduce: read the sender's and the receiver's element,
// write the receiver's; copy: read the sender's, write the receiver's), so
// the counted bytes are the stepwise ones, 5 (P-1) s per element.
//
// With the chain c[0..P) of the span in groups of C = `group` entries
// (G = P / C groups; rings have one group of P):
//   row reduce-scatter of each group g: c[gC+t+1] (+)= c[gC+t], t = 0..C-2
//   column reduce-scatter: c[(t+1)C+C-1] (+)= c[tC+C-1], t = 0..G-2
//   column all-gather: c[tC+C-1] = c[((t-1) mod G)C+C-1], t = 0..G-2
//   row all-gather of each group: c[gC+t] = c[gC+(t-1) mod C], t = 0..C-2
// with the mean fused into the add that completes the sum (the last column
// add, or the last row add when G = 1).  For a ring, position x of the ring
// is chain entry (x - c) mod P of chunk c, so these are the ring's steps;
// for the torus, group g is row (d + g) mod rows of sub-piece d, and its
// last entry is the rank of column (c - 1) mod cols that owns row piece c.
// ---------------------------------------------------------------------------
template <class V>
__device__ __forceinline__ V ld_at(uint64_t addr) {
    return *reinterpret_cast<const V DDL_STEP_GLOBAL *>(addr);
}
template <class V>
__device__ __forceinline__ void st_at(uint64_t addr, V v) {
    *reinterpret_cast<V DDL_STEP_GLOBAL *>(addr) = v;
}

// The SGD step riding on the walk (null for the plain all-reduce): weight
// replica addresses in chain order (every entry replica 0 when one replica
// is shared), the rate, and whether the replica is shared.
struct WalkSgd {
    const uint64_t *w;
    float lr;
    bool shared;
};

// The walk of U values of type X (vectors, or single elements with U = 1)
// at byte offsets off + u * stride of every rank, rank addresses in chain
// order in c[].  With kSgd, each rank's weights (binary32, at element
// offsets off / sizeof(T)) take their step where the reduced value reaches
// the rank: chain entry P - 1 at the add that completes the sum, every other
// entry when an all-gather copy delivers it (with one shared replica, entry
// P - 1 alone) -- the ranks and values of the per-step launches.
template <class E, class X, int U, bool kSgd = false>
__device__ __forceinline__ void walk_body(const uint64_t *c, int P, int C, bool mean,
                                          float divisor, uint64_t off, uint64_t stride,
                                          const WalkSgd *sgd = nullptr) {
    using T = typename E::T;
    constexpr bool kVec = sizeof(X) == sizeof(typename E::V);
    using Wx = typename std::conditional<kVec, typename E::W, float>::type;
    const int G = P / C;
    // the weights of chain entry dst take their step with the values r
    auto update = [&](int dst, const X (&r)[U]) {
        if constexpr (kSgd) {
            if (sgd->shared && dst != P - 1)
                return;
            const uint64_t wo = off / sizeof(T) * sizeof(float);
            const uint64_t ws = stride / sizeof(T) * sizeof(float);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint64_t wa = sgd->w[dst] + wo + u * ws;
                Wx y;
                if constexpr (kVec)
                    y = E::widen(r[u]);
                else
                    y = (float)r[u];
                st_at<Wx>(wa, sgd_step<Wx>(ld_at<Wx>(wa), y, sgd->lr));
            }
        }
    };
    auto add = [](X a, X b) {
        if constexpr (sizeof(X) == sizeof(typename E::V))
            return E::add(a, b);
        else
            return E::add1(a, b);
    };
    auto div = [](X a, float d) {
        if constexpr (sizeof(X) == sizeof(typename E::V))
            return E::div(a, d);
        else
            return E::div1(a, d);
    };
    // reduce: dst (+)= src; the add that completes the sum (fin) also
    // divides by P for the mean and takes the owner's SGD step
    auto reduce = [&](int src, int dst, bool fin) {
        X s[U], d[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            s[u] = ld_at<X>(c[src] + off + u * stride);
            d[u] = ld_at<X>(c[dst] + off + u * stride);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            d[u] = add(d[u], s[u]);
            if (fin && mean)
                d[u] = div(d[u], divisor);
            st_at<X>(c[dst] + off + u * stride, d[u]);
        }
        if (fin)
            update(dst, d);
    };
    auto copy = [&](int src, int dst) {
        X s[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            s[u] = ld_at<X>(c[src] + off + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u)
            st_at<X>(c[dst] + off + u * stride, s[u]);
        update(dst, s);
    };
    for (int g = 0; g < G; ++g)
        for (int t = 0; t + 1 < C; ++t)
            reduce(g * C + t, g * C + t + 1, G == 1 && t == C - 2);
    for (int t = 0; t + 1 < G; ++t)
        reduce(t * C + C - 1, (t + 1) * C + C - 1, t == G - 2);
    for (int t = 0; t + 1 < G; ++t)
        copy(((t + G - 1) % G) * C + C - 1, t * C + C - 1);
    for (int g = 0; g < G; ++g)
        for (int t = 0; t + 1 < C; ++t)
            copy(g * C + (t + C - 1) % C, g * C + t);
}

// Workgroup b walks tile tile_base + b of the fused span table (with kSgd,
// taking the SGD step of g on the way).
template <class E, bool kSgd>
__device__ __forceinline__ void walk_tile(const RankPtrs &bufs, const FusedArgs &a,
                                          const SgdArgs *g) {
    using T = typename E::T;
    using V = typename E::V;
    constexpr int U = fused_vecs_per_lane(sizeof(T));
    constexpr uint64_t kTile = fused_tile_elems(sizeof(T));
    constexpr uint64_t kStride = (uint64_t)kBlock * E::N * sizeof(T);
    __shared__ uint64_t c[DDL_MAX_RANKS];   // rank addresses, chain order
    __shared__ uint64_t wc[kSgd ? DDL_MAX_RANKS : 1];  // their weight replicas
    const int P = a.P;
    const uint32_t tid = threadIdx.x;
    const uint32_t tile = a.tile_base + blockIdx.x;
    const uint32_t i = a.tile_span[tile];
    const DevSpan sp = a.spans[i];
    for (int j = (int)tid; j < P; j += kBlock) {
        const int r = a.chains[sp.chain_off + j];
        c[j] = reinterpret_cast<uint64_t>(bufs.p[r]);
        if (kSgd)
            wc[j] = reinterpret_cast<uint64_t>(g->w.p[g->nweights == 1 ? 0 : r]);
    }
    __syncthreads();
    WalkSgd ws{wc, kSgd ? g->lr : 0.0f, kSgd && g->nweights == 1};
    const WalkSgd *wsp = kSgd ? &ws : nullptr;
    const uint64_t j = tile - a.prefix[i];
    const uint64_t sh = tile_shift(sp.off, kTile, a.anchor);
    const uint64_t base = tile_lo(sp.off, sh, kTile, j);
    const uint32_t cnt = (uint32_t)(tile_hi(sp.off, sp.len, sh, kTile, j) - base);
    const bool mean = a.mean != 0;
    uint32_t done = 0;
    if (sp.flags & kItemAligned) {
        const uint32_t nvec = cnt / E::N;
        if (nvec == (uint32_t)(U * kBlock)) {
            walk_body<E, V, U, kSgd>(c, P, a.group, mean, a.divisor,
                                     (base + (uint64_t)tid * E::N) * sizeof(T), kStride, wsp);
        } else {
            for (uint32_t v = tid; v < nvec; v += kBlock)
                walk_body<E, V, 1, kSgd>(c, P, a.group, mean, a.divisor,
                                         (base + (uint64_t)v * E::N) * sizeof(T), 0, wsp);
        }
        done = nvec * E::N;
    }
    for (uint32_t k = done + tid; k < cnt; k += kBlock)
        walk_body<E, T, 1, kSgd>(c, P, a.group, mean, a.divisor, (base + k) * sizeof(T), 0,
                                 wsp);
}

template <class E>
__global__ __launch_bounds__(kBlock) void walk_kernel(RankPtrs bufs, FusedArgs a) {
    walk_tile<E, false>(bufs, a, nullptr);
}

template <class E>
__global__ __launch_bounds__(kBlock) void walk_sgd_kernel(RankPtrs bufs, FusedArgs a,
                                                          SgdArgs g) {
    walk_tile<E, true>(bufs, a, &g);
}

}  // namespace

namespace {

template <class E, int VPL>
void launch_v(int kind, dim3 grid, hipStream_t s, const RankPtrs &bufs, const StepArgs &a,
              const SgdArgs *sgd) {
    const dim3 block(kBlock);
    if (sgd) {
        if (kind == DDL_K_REDUCE)
            hipLaunchKernelGGL((step_sgd_kernel<E, true, VPL>), grid, block, 0, s, bufs, a,
                               *sgd);
        else
            hipLaunchKernelGGL((step_sgd_kernel<E, false, VPL>), grid, block, 0, s, bufs, a,
                               *sgd);
        return;
    }
    if (kind == DDL_K_REDUCE)
        hipLaunchKernelGGL((step_kernel<E, true, VPL>), grid, block, 0, s, bufs, a);
    else
        hipLaunchKernelGGL((step_kernel<E, false, VPL>), grid, block, 0, s, bufs, a);
}

template <class E>
void launch_e(int kind, int vpl, dim3 grid, hipStream_t s, const RankPtrs &bufs,
              const StepArgs &a, const SgdArgs *sgd) {
    if (vpl == 1)
        launch_v<E, 1>(kind, grid, s, bufs, a, sgd);
    else if (vpl == 2)
        launch_v<E, 2>(kind, grid, s, bufs, a, sgd);
    else
        launch_v<E, 4>(kind, grid, s, bufs, a, sgd);
}

}  // namespace

int launch_walk(int dtype, const RankPtrs &bufs, const FusedArgs &a, const SgdArgs *sgd,
                uint32_t tiles, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (tiles == 0)
        return (int)hipSuccess;
    const dim3 grid(tiles), block(kBlock);
    if (sgd) {
        if (dtype == DDL_F32)
            hipLaunchKernelGGL((walk_sgd_kernel<F32>), grid, block, 0, s, bufs, a, *sgd);
        else
            hipLaunchKernelGGL((walk_sgd_kernel<F16>), grid, block, 0, s, bufs, a, *sgd);
    } else if (dtype == DDL_F32) {
        hipLaunchKernelGGL((walk_kernel<F32>), grid, block, 0, s, bufs, a);
    } else {
        hipLaunchKernelGGL((walk_kernel<F16>), grid, block, 0, s, bufs, a);
    }
    return (int)hipGetLastError();
}

int launch_step(int dtype, int kind, int vpl, const RankPtrs &bufs, const StepArgs &a,
                const SgdArgs *sgd, uint32_t tiles, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == DDL_F32)
        launch_e<F32>(kind, vpl, dim3(tiles), s, bufs, a, sgd);
    else
        launch_e<F16>(kind, vpl, dim3(tiles), s, bufs, a, sgd);
    return (int)hipGetLastError();
}

}  // namespace ddl
