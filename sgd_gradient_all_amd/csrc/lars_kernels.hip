// lars_kernels.hip -- the LARS step after the all-reduce (gfx950).
//
// The Sony ResNet-50 article ("训练设置") updates the weights with LARS,
// coefficient 0.01 and eps 1e-6: the layer-wise adaptive rate scaling of
// You, Gitman and Ginsburg, whose formula the page does not carry.  Each
// layer -- here each bucket -- gets the learning rate lr * trust with
//     trust = coeff * ||w|| / (||y|| + eps)    (1 when ||w|| or ||y|| is 0),
// the norms taken over the layer from replica 0's weights (replicas of a
// synchronous step are identical) and the all-reduced gradient y; no weight
// decay or momentum is stated, so none is applied.  Then every replica takes
// the SGD step w - rate * y.
//
// A layer's rate needs the whole layer reduced first, so the step cannot
// ride in the all-reduce's epilogue as plain SGD does.  In the fused pass's
// two-kernel form the norms ride in the reduce kernel (each workgroup sums
// the squares of its tile of y and w_0) and the update in the broadcast
// (fused_kernel.hip), with lars_rate_kernel between them over the fused
// tiles' partial sums.  Otherwise, per bucket group, after its all-reduce,
// three launches over the buckets' anchored tiles:
//  - lars_norm_kernel: one workgroup per tile sums w_0[e]^2 and y[e]^2 in
//    binary64 (each square of a binary32 value is exact there) and writes
//    the two partial sums of the tile;
//  - lars_rate_kernel: one workgroup per bucket adds its tiles' partials
//    and writes rate = binary32(lr * trust), trust in binary64;
//  - update_kernel: each tile takes ceil(nweights / G) workgroups, each
//    loading y and stepping G replicas with the bucket's rate (G = 2 by
//    default: measured on MI355X with 40 replicas, 8% faster than one
//    workgroup stepping all of them; the extra loads of y hit the cache).
// HBM: the norms read y and w_0 (s + 4 bytes per element), the update reads
// y and reads and writes every replica (s + 8 nweights); the partials are
// 16 bytes per tile.  Both streaming kernels are HBM-bound.  Measured with
// rocprofv3 counters on MI355X (40 replicas): the norm kernel moves 1.01x
// its bytes, the update kernel 1.09x -- each accelerator die fetches y once
// for the replica groups of a tile that run on it.
//
// The sums' association order (per lane in element order, then a fixed
// tree over the workgroup, then the tiles of a bucket in a fixed tree) is
// deterministic from run to run but is not the oracle's index order, so
// rates agree with it to the binary64 rounding of the norms: equal in
// binary32 except where lr * trust falls within ~1e-13 of a rounding
// boundary.
#include "device_common.h"

#include <map>
#include <mutex>

namespace ddl {

// The fixed scratch of the allocation-free LARS entry point: per-tile
// partial sums (16 bytes per tile) and per-bucket rates (4 bytes each) for
// callers that cannot allocate.  Each device holds its own copy at its own
// address; host code reaches it only through the address hipGetSymbolAddress
// gives for that device (lars_scratch below), never through this name.
static __device__ __align__(256) unsigned char scratch[kLarsScratchBytes];

namespace {

using namespace dev;

#define DDL_LARS_GLOBAL __attribute__((address_space(1)))

template <class V>
__device__ __forceinline__ V ld_nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const V *>(p));
}
template <class V>
__device__ __forceinline__ void st_nt(void *p, V v) {
    __builtin_nontemporal_store(v, reinterpret_cast<V *>(p));
}

// Elements [base, base + cnt) of tile t of the bucket table, and whether
// they are 16-byte aligned.  Uniform across the workgroup.
struct TileRange {
    uint64_t base;
    uint32_t cnt;
    uint32_t bucket;
    bool aligned;
};

template <int kEsz>
__device__ __forceinline__ TileRange tile_range(const LarsArgs &a, uint32_t t) {
    constexpr uint64_t kTile = fused_tile_elems(kEsz);
    TileRange r;
    r.bucket = a.tile_span[t];
    const DevSpan sp = a.spans[r.bucket];
    const uint64_t j = t - a.prefix[r.bucket];
    const uint64_t sh = tile_shift(sp.off, kTile, true);
    r.base = tile_lo(sp.off, sh, kTile, j);
    r.cnt = (uint32_t)(tile_hi(sp.off, sp.len, sh, kTile, j) - r.base);
    r.aligned = (sp.flags & kItemAligned) != 0;
    return r;
}


// ---------------------------------------------------------------------------
// norms: workgroup b sums the squares of tile tile_base + b
// ---------------------------------------------------------------------------
template <class E>
__global__ __launch_bounds__(kBlock) void lars_norm_kernel(RankPtrs w, LarsArgs a) {
    using T = typename E::T;
    using V = typename E::V;
    using Wv = typename E::W;
    constexpr int U = fused_vecs_per_lane(sizeof(T));
    constexpr uint64_t kStride = (uint64_t)kBlock * E::N;
    __shared__ double lds[2][kBlock / 64];
    const uint32_t t = a.tile_base + blockIdx.x;
    const TileRange tr = tile_range<sizeof(T)>(a, t);
    const T *y = static_cast<const T *>(a.y);
    const float *w0 = static_cast<const float *>(w.p[0]);
    const uint32_t tid = threadIdx.x;
    double sw = 0.0, sy = 0.0;
    uint32_t done = 0;
    if (tr.aligned) {
        const uint32_t nvec = tr.cnt / E::N;
        if (nvec == (uint32_t)(U * kBlock)) {
            const uint64_t e = tr.base + (uint64_t)tid * E::N;
            V yv[U];
            Wv wv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                yv[u] = ld_nt<V>(y + e + u * kStride);
                wv[u] = ld_nt<Wv>(w0 + e + u * kStride);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                add_squares<Wv>(E::widen(yv[u]), sy);
                add_squares<Wv>(wv[u], sw);
            }
        } else {
            for (uint32_t k = tid; k < nvec; k += kBlock) {
                const uint64_t e = tr.base + (uint64_t)k * E::N;
                add_squares<Wv>(E::widen(ld_nt<V>(y + e)), sy);
                add_squares<Wv>(ld_nt<Wv>(w0 + e), sw);
            }
        }
        done = nvec * E::N;
    }
    for (uint32_t k = done + tid; k < tr.cnt; k += kBlock) {
        const uint64_t e = tr.base + k;
        const double g = (double)(float)y[e], x = (double)w0[e];
        sy += g * g;
        sw += x * x;
    }
    const double tw = block_sum(sw, lds[0]);
    const double ty = block_sum(sy, lds[1]);
    if (tid == 0) {
        a.partial[2 * (uint64_t)t] = tw;
        a.partial[2 * (uint64_t)t + 1] = ty;
    }
}

// ---------------------------------------------------------------------------
// rates: workgroup b adds the partials of bucket bucket_lo + b
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void lars_rate_kernel(LarsArgs a) {
    __shared__ double lds[2][kBlock / 64];
    const uint32_t i = a.bucket_lo + blockIdx.x;
    const uint32_t t0 = a.prefix[i], t1 = a.prefix[i + 1];
    // each lane adds tiles t0 + lane, t0 + lane + kBlock, ... in that order;
    // kU of them are loaded ahead of their adds (a bucket of the 300M-element
    // workload has ~4600 tiles: one round of loads per kU instead of per tile)
    constexpr uint32_t kU = 8;
    double sw = 0.0, sy = 0.0;
    uint32_t t = t0 + threadIdx.x;
    for (; t + (kU - 1) * kBlock < t1; t += kU * kBlock) {
        double pw[kU], py[kU];
#pragma unroll
        for (uint32_t u = 0; u < kU; ++u) {
            pw[u] = a.partial[2 * (uint64_t)(t + u * kBlock)];
            py[u] = a.partial[2 * (uint64_t)(t + u * kBlock) + 1];
        }
#pragma unroll
        for (uint32_t u = 0; u < kU; ++u) {
            sw += pw[u];
            sy += py[u];
        }
    }
    for (; t < t1; t += kBlock) {
        sw += a.partial[2 * (uint64_t)t];
        sy += a.partial[2 * (uint64_t)t + 1];
    }
    const double W = block_sum(sw, lds[0]);
    const double G = block_sum(sy, lds[1]);
    if (threadIdx.x == 0) {
        double trust = 1.0;
        if (W > 0.0 && G > 0.0)
            trust = a.coeff * sqrt(W) / (sqrt(G) + a.eps);
        const float rate = (float)((double)a.lr * trust);
        a.rate[i] = rate;
        if (a.rate_out)
            a.rate_out[i] = rate;
    }
}

// ---------------------------------------------------------------------------
// update: workgroup b steps replicas [g * G, (g + 1) * G) over tile
// tile_base + b / ngroups, g = b % ngroups, G = reps_per_group.  The
// replicas go in batches of kRB: every load of a batch is issued before its
// stores, so a wave keeps kRB requests in flight.
// ---------------------------------------------------------------------------
template <class E, int kRB>
__global__ __launch_bounds__(kBlock) void update_kernel(RankPtrs w, LarsArgs a) {
    using T = typename E::T;
    using V = typename E::V;
    using Wv = typename E::W;
    constexpr int U = fused_vecs_per_lane(sizeof(T));
    constexpr uint64_t kStride = (uint64_t)kBlock * E::N;
    const uint32_t ng = (uint32_t)a.ngroups;
    const uint32_t t = a.tile_base + blockIdx.x / ng;
    const int rb = (int)(blockIdx.x % ng) * a.reps_per_group;
    const int nw = min(a.nweights, rb + a.reps_per_group);
    const TileRange tr = tile_range<sizeof(T)>(a, t);
    const float rate = a.rate ? a.rate[tr.bucket] : a.lr;
    const T *y = static_cast<const T *>(a.y);
    const uint32_t tid = threadIdx.x;
    uint32_t done = 0;
    if (tr.aligned) {
        const uint32_t nvec = tr.cnt / E::N;
        if (nvec == (uint32_t)(U * kBlock)) {
            const uint64_t e = tr.base + (uint64_t)tid * E::N;
            Wv g[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                g[u] = E::widen(ld_nt<V>(y + e + u * kStride));
            for (int r0 = rb; r0 < nw; r0 += kRB) {
                Wv x[kRB][U];
#pragma unroll
                for (int k = 0; k < kRB; ++k)
                    if (r0 + k < nw)
#pragma unroll
                        for (int u = 0; u < U; ++u)
                            x[k][u] = ld_nt<Wv>(static_cast<const float *>(w.p[r0 + k]) + e +
                                                u * kStride);
#pragma unroll
                for (int k = 0; k < kRB; ++k)
                    if (r0 + k < nw)
#pragma unroll
                        for (int u = 0; u < U; ++u)
                            st_nt<Wv>(static_cast<float *>(w.p[r0 + k]) + e + u * kStride,
                                      sgd_step<Wv>(x[k][u], g[u], rate));
            }
        } else {
            for (uint32_t k = tid; k < nvec; k += kBlock) {
                const uint64_t e = tr.base + (uint64_t)k * E::N;
                const Wv g = E::widen(ld_nt<V>(y + e));
                for (int r = rb; r < nw; ++r) {
                    float *wp = static_cast<float *>(w.p[r]) + e;
                    st_nt<Wv>(wp, sgd_step<Wv>(ld_nt<Wv>(wp), g, rate));
                }
            }
        }
        done = nvec * E::N;
    }
    for (uint32_t k = done + tid; k < tr.cnt; k += kBlock) {
        const uint64_t e = tr.base + k;
        const float g = (float)y[e];
        for (int r = rb; r < nw; ++r) {
            float *wp = static_cast<float *>(w.p[r]) + e;
            *wp = sgd_step<float>(*wp, g, rate);
        }
    }
}

template <class E>
void launch_update(dim3 grid, hipStream_t s, const RankPtrs &w, const LarsArgs &a, int batch) {
    const dim3 block(kBlock);
    switch (batch) {
    case 1: hipLaunchKernelGGL((update_kernel<E, 1>), grid, block, 0, s, w, a); break;
    case 2: hipLaunchKernelGGL((update_kernel<E, 2>), grid, block, 0, s, w, a); break;
    case 8: hipLaunchKernelGGL((update_kernel<E, 8>), grid, block, 0, s, w, a); break;
    default: hipLaunchKernelGGL((update_kernel<E, 4>), grid, block, 0, s, w, a); break;
    }
}

}  // namespace

int lars_scratch(int device, void **ptr, size_t *bytes) {
    static std::mutex mu;
    static std::map<int, void *> &addr = *new std::map<int, void *>;
    std::lock_guard<std::mutex> lk(mu);
    auto it = addr.find(device);
    if (it == addr.end()) {
        // once per device, with that device current
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess)
            return (int)e;
        if (cur != device && (e = hipSetDevice(device)) != hipSuccess)
            return (int)e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != device)
            (void)hipSetDevice(cur);
        if (e != hipSuccess || !p)
            return (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
        it = addr.emplace(device, p).first;
    }
    *ptr = it->second;
    *bytes = kLarsScratchBytes;
    return (int)hipSuccess;
}

int launch_lars(int dtype, int kind, const RankPtrs &w, const LarsArgs &a, uint32_t blocks,
                void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (blocks == 0)
        return (int)hipSuccess;
    const dim3 grid(blocks), block(kBlock);
    switch (kind) {
    case DDL_K_LARS_NORM:
        if (dtype == DDL_F32)
            hipLaunchKernelGGL((lars_norm_kernel<F32>), grid, block, 0, s, w, a);
        else
            hipLaunchKernelGGL((lars_norm_kernel<F16>), grid, block, 0, s, w, a);
        break;
    case DDL_K_LARS_RATE:
        hipLaunchKernelGGL(lars_rate_kernel, grid, block, 0, s, a);
        break;
    case DDL_K_UPDATE: {
        // blocks counts tiles; every tile takes ngroups workgroups, and a
        // grid holds at most 2^32 - 1 work-items: cut into several launches
        if (a.ngroups < 1 || a.reps_per_group < 1)
            return (int)hipErrorInvalidValue;
        const uint32_t per = 0xffffffffu / (uint32_t)kBlock / (uint32_t)a.ngroups;
        if (per == 0)
            return (int)hipErrorInvalidValue;
        const int batch = tuning(DDL_TUNE_UPDATE_BATCH);
        for (uint32_t t0 = 0; t0 < blocks; t0 += per) {
            LarsArgs b = a;
            b.tile_base = a.tile_base + t0;
            const dim3 ugrid(min(per, blocks - t0) * (uint32_t)a.ngroups);
            if (dtype == DDL_F32)
                launch_update<F32>(ugrid, s, w, b, batch);
            else
                launch_update<F16>(ugrid, s, w, b, batch);
        }
        break;
    }
    default:
        return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

}  // namespace ddl
