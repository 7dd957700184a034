// fused_kernel.hip -- the fused all-reduce pass (gfx950).
//
// Every element is read once from each of the P ranks, summed in the order
// the schedule sums it, divided by P for the mean, and written once to each
// rank: 2 P s bytes per element, the floor for this operation.  It is
// bit-identical to the step-by-step walk because every dependency of the
// schedule is per element.
//
// The pass runs in one of two forms:
//  - one kernel (fused_kernel): each workgroup reads its tile from all P
//    ranks and writes the result to all P ranks;
//  - two kernels over the same tiles: the reduce kernel reads all P ranks
//    and writes the result to rank 0 only (or, for an SGD step that leaves
//    the gradients as they were, to a scratch buffer), through the cache --
//    rank by rank over 4 or 6 tiles per workgroup from 16 ranks on
//    (fused_reduce_ranks_kernel), tile by tile below (fused_reduce_kernel);
//    then bcast_kernel copies rank 0's result, still cache-resident, to
//    ranks 1..P-1.  HBM then sees a read phase and a write phase instead of
//    reads and writes interleaved.  Measured on MI355X in paired runs: 40
//    ranks binary32 +5..+18% (the spread is the physical placement of the
//    buffers, to which the two-kernel form is far less sensitive), 16 ranks
//    binary16 +5%, 16 ranks binary32 -3..+7%, 8 ranks -3%.  Plans choose
//    the form (plan.cpp, fused_passes).
//
// Writes: stores are non-temporal, and a wave that stores to several ranks
// may wait for each rank's stores to complete before the next (the
// broadcast in binary32, the one-kernel pass in large binary32 groups; see
// bcast_store_wait, fused_store_wait).
#include "device_common.h"

namespace ddl {
namespace {

using namespace dev;

// Streaming accesses.  Every element is touched once per pass, so the
// results are written with non-temporal stores.  In the one-kernel form,
// loads are non-temporal when P times the elements a lane loads per rank is
// at most 4 x 24 (knob DDL_TUNE_FUSED_NT_LOAD_MAX_P): up to 24 binary32
// ranks, 12 binary16 ranks.  Measured on MI355X: +7..+15% for binary32 at 8
// and 16 ranks and binary16 at 8, -4% for binary32 at 40 ranks; binary16 at
// 12-16 ranks either way by size (-7..+10%).
#ifndef DDL_NT_STORE
#define DDL_NT_STORE 1
#endif
// Loads a lane issues ahead of their adds in the tile-by-tile walks (kB,
// 1, 2, 4 or 8; knobs DDL_TUNE_FUSED_BATCH and DDL_TUNE_REDUCE_BATCH).
// The adds stay in chain order; a batch only lets a wave keep kB requests
// in flight instead of waiting for each load before issuing the next.
// Measured on MI355X: the read-only reduce kernel tile by tile gains from 4
// (+4.6% at 40 ranks, +2% at 16); the one-kernel pass, whose writes share
// HBM with the reads, is best with 1 at 8 ranks (2: -1%, 4: -3.5%).  The
// rank-by-rank reduce issues its loads two at a time (kReduceIssue).
// Waves per SIMD the register allocation must allow: 8 for one vector per
// lane (no spills at 56 VGPRs), 4 for two.
#ifndef DDL_FUSED_WAVES_1
#define DDL_FUSED_WAVES_1 8
#endif
#ifndef DDL_FUSED_WAVES_2
#define DDL_FUSED_WAVES_2 4
#endif

template <class V, bool kNt>
__device__ __forceinline__ V ld_stream(const void *p) {
    if (kNt)
        return __builtin_nontemporal_load(reinterpret_cast<const V *>(p));
    return *reinterpret_cast<const V *>(p);
}

// The rank streams are read through global (address space 1) pointers built
// from addresses kept in LDS.  A generic pointer would compile to FLAT
// loads, which also count against the LDS wait counter: every wait for the
// next address would then wait for all data loads in flight.
#define DDL_GLOBAL __attribute__((address_space(1)))
template <class V, bool kNt>
__device__ __forceinline__ V ld_global(uint64_t addr) {
    const V DDL_GLOBAL *p = reinterpret_cast<const V DDL_GLOBAL *>(addr);
    if (kNt)
        return __builtin_nontemporal_load(p);
    return *p;
}
// Wait until this wave's memory operations in flight, its stores included,
// have completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <class V>
__device__ __forceinline__ void st_stream(void *p, V v) {
#if DDL_NT_STORE
    __builtin_nontemporal_store(v, reinterpret_cast<V *>(p));
#else
    *reinterpret_cast<V *>(p) = v;
#endif
}

// ---------------------------------------------------------------------------
// fused pass: every element is read once from each of the P ranks, summed in
// the order the schedule sums it -- chain[0..P) in groups of `group`
// entries, each group left to right, then the group sums left to right --
// divided by P for the mean, and written once to each rank.
//
// The rank addresses, in chain order, are staged in LDS before the first
// load, so the data loads never wait behind a table load.
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

// Sums of U element vectors -- e + u * kBlock * N, u < U -- over the chain.
// The ranks go in batches of kB from the first one; every load of a
// batch is issued before the batch's adds.  In a partial last batch the
// missing slots re-load the batch's last rank (a line already in flight) and
// their adds are skipped, which keeps every load unconditional.  Ungrouped (rings): one
// chain of P entries.  Grouped (torus): chains of `group` entries, then
// their sums.
template <class E, bool kGrouped, bool kNt, int U, int kB>
__device__ __forceinline__ void fused_vecs(const uint64_t *sp, int P, int group,
                                           uint64_t e, typename E::V (&out)[U]) {
    using V = typename E::V;
    constexpr uint64_t kStride = (uint64_t)kBlock * E::N;
    Chain<E> c[U];
    V acc[U];
    for (int b = 0; b < P; b += kB) {
        const int nb = min(kB, P - b);
        V x[kB][U];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            const uint64_t p = sp[b + (j < nb ? j : nb - 1)] + e * sizeof(typename E::T);
#pragma unroll
            for (int u = 0; u < U; ++u)
                x[j][u] = ld_global<V, kNt>(p + u * kStride * sizeof(typename E::T));
        }
#pragma unroll
        for (int j = 0; j < kB; ++j)
            if (j < nb)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (kGrouped)
                        c[u].push(x[j][u], group);
                    else
                        acc[u] = b + j == 0 ? x[j][u] : E::add(acc[u], x[j][u]);
                }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
        out[u] = kGrouped ? c[u].acc : acc[u];
}

template <class E, int U, bool kWait = false>
__device__ __forceinline__ void store_all(const RankPtrs &bufs, int P, uint64_t e,
                                          const typename E::V (&v)[U]) {
    using T = typename E::T;
    constexpr uint64_t kStride = (uint64_t)kBlock * E::N;
    for (int r = 0; r < P; ++r) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            st_stream<typename E::V>(static_cast<T *>(bufs.p[r]) + e + u * kStride, v[u]);
        if (kWait)
            wait_stores();
    }
}

// The SGD step of every weight replica on the reduced vectors v[0..U) of
// element e (binary32 weights; non-temporal like the rest of the pass).
template <class E, bool kNt, int U>
__device__ __forceinline__ void sgd_all(const SgdArgs *g, uint64_t e,
                                        const typename E::V (&v)[U]) {
    using W = typename E::W;
    constexpr uint64_t kStride = (uint64_t)kBlock * E::N;
    for (int r = 0; r < g->nweights; ++r)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float *wp = static_cast<float *>(g->w.p[r]) + e + u * kStride;
            st_stream<W>(wp, sgd_step<W>(ld_stream<W, kNt>(wp), E::widen(v[u]), g->lr));
        }
}

// Stores of the reduced vectors v[0..U) of element e to the home buffer
// only (rank 0's, or a scratch buffer when the gradients must stay as they
// were), with ordinary (cached) stores: the kernel that follows re-reads
// them.
template <class E, int U>
__device__ __forceinline__ void store_home(void *home, uint64_t e,
                                           const typename E::V (&v)[U]) {
    using T = typename E::T;
    using V = typename E::V;
    constexpr uint64_t kStride = (uint64_t)kBlock * E::N;
    V DDL_GLOBAL *h = reinterpret_cast<V DDL_GLOBAL *>(
        reinterpret_cast<uint64_t>(home) + e * sizeof(T));
#pragma unroll
    for (int u = 0; u < U; ++u)
        h[u * (kStride / E::N)] = v[u];
}

// kHome: write the result to the home buffer only (the first kernel of the
// two-kernel form); otherwise to every rank.  kLars (with kHome): also the
// LARS step's norms -- per tile, the binary64 sums of the squares of the
// result y and of replica 0's weights w0, each lane in element order, then
// over the workgroup (block_sum), written to a.partial[2t] (w0) and
// a.partial[2t + 1] (y).
template <class E, bool kGrouped, bool kNt, bool kSgd, bool kHome, int kB, bool kLars = false,
          bool kWait = false>
__device__ __forceinline__ void fused_body(const RankPtrs &bufs, const FusedArgs &a,
                                           const SgdArgs *g) {
    using T = typename E::T;
    using V = typename E::V;
    using Wv = typename E::W;
    constexpr int U = fused_vecs_per_lane(sizeof(T));
    constexpr uint64_t kTile = fused_tile_elems(sizeof(T));
    constexpr uint64_t kStride = (uint64_t)kBlock * E::N;
    __shared__ uint64_t src[DDL_MAX_RANKS];  // rank stream addresses, chain order
    __shared__ double lds_norm[2][kBlock / 64];
    const int P = a.P;
    const uint32_t tid = threadIdx.x;
    const uint32_t first = a.tile_base + blockIdx.x * (uint32_t)kFusedTilesPerGroup;
    const uint32_t last = min(first + (uint32_t)kFusedTilesPerGroup, a.tile_end);
    uint32_t i = a.span_lo, have = UINT32_MAX;
    for (uint32_t tile = first; tile < last; ++tile) {
        i = a.tile_span[tile];
        const DevSpan sp = a.spans[i];
        if (i != have) {
            // a new span: its chain decides which rank is read first
            if (have != UINT32_MAX)
                __syncthreads();
            for (int j = (int)tid; j < P; j += kBlock)
                src[j] = reinterpret_cast<uint64_t>(bufs.p[a.chains[sp.chain_off + j]]);
            __syncthreads();
            have = i;
        }
        const uint64_t j = tile - a.prefix[i];
        const uint64_t sh = tile_shift(sp.off, kTile, a.anchor);
        const uint64_t base = tile_lo(sp.off, sh, kTile, j);
        const uint32_t cnt = (uint32_t)(tile_hi(sp.off, sp.len, sh, kTile, j) - base);
        uint32_t done = 0;
        double sw = 0.0, sy = 0.0;  // kLars: this lane's sums of squares
        if (sp.flags & kItemAligned) {
            const uint32_t nvec = cnt / E::N;
            if (nvec == (uint32_t)(U * kBlock)) {
                const uint64_t e = base + (uint64_t)tid * E::N;
                V acc[U];
                fused_vecs<E, kGrouped, kNt, U, kB>(src, P, a.group, e, acc);
                if (a.mean)
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        acc[u] = E::div(acc[u], a.divisor);
                if (kHome)
                    store_home<E, U>(a.home, e, acc);
                else if (!kSgd || g->keep_grads)
                    store_all<E, U, kWait>(bufs, P, e, acc);
                if (kSgd)
                    sgd_all<E, kNt, U>(g, e, acc);
                if (kLars) {
                    Wv wv[U];
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        wv[u] = ld_stream<Wv, true>(a.w0 + e + u * kStride);
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        add_squares<Wv>(E::widen(acc[u]), sy);
                        add_squares<Wv>(wv[u], sw);
                    }
                }
            } else {
                for (uint32_t v = tid; v < nvec; v += kBlock) {
                    const uint64_t e = base + (uint64_t)v * E::N;
                    V acc[1];
                    fused_vecs<E, kGrouped, kNt, 1, kB>(src, P, a.group, e, acc);
                    if (a.mean)
                        acc[0] = E::div(acc[0], a.divisor);
                    if (kHome)
                        store_home<E, 1>(a.home, e, acc);
                    else if (!kSgd || g->keep_grads)
                        store_all<E, 1, kWait>(bufs, P, e, acc);
                    if (kSgd)
                        sgd_all<E, kNt, 1>(g, e, acc);
                    if (kLars) {
                        add_squares<Wv>(E::widen(acc[0]), sy);
                        add_squares<Wv>(ld_stream<Wv, true>(a.w0 + e), sw);
                    }
                }
            }
            done = nvec * E::N;
        }
        for (uint32_t k = done + tid; k < cnt; k += kBlock) {
            const uint64_t e = base + k;
            T acc = 0, gacc = 0;
            int pos = 0;
            bool first_group = true;
            for (int j = 0; j < P; ++j) {
                T x = *reinterpret_cast<const T DDL_GLOBAL *>(src[j] + e * sizeof(T));
                gacc = pos == 0 ? x : E::add1(gacc, x);
                if (++pos == a.group) {
                    acc = first_group ? gacc : E::add1(acc, gacc);
                    first_group = false;
                    pos = 0;
                }
            }
            if (a.mean)
                acc = E::div1(acc, a.divisor);
            if (kHome)
                static_cast<T *>(a.home)[e] = acc;
            else if (!kSgd || g->keep_grads)
                for (int r = 0; r < P; ++r)
                    static_cast<T *>(bufs.p[r])[e] = acc;
            if (kSgd)
                for (int r = 0; r < g->nweights; ++r) {
                    float *wp = static_cast<float *>(g->w.p[r]) + e;
                    *wp = sgd_step<float>(*wp, (float)acc, g->lr);
                }
            if (kLars) {
                const double y = (double)(float)acc, x = (double)a.w0[e];
                sy += y * y;
                sw += x * x;
            }
        }
        if (kLars) {
            const double tw = block_sum(sw, lds_norm[0]);
            const double ty = block_sum(sy, lds_norm[1]);
            if (tid == 0) {
                a.partial[2 * (uint64_t)tile] = tw;
                a.partial[2 * (uint64_t)tile + 1] = ty;
            }
            __syncthreads();  // lds_norm is read before the next tile's sums
        }
    }
}

#define DDL_FUSED_OCCUPANCY                                                      \
    __attribute__((amdgpu_waves_per_eu(fused_vecs_per_lane(sizeof(typename E::T)) == 1 \
                                           ? DDL_FUSED_WAVES_1                        \
                                           : DDL_FUSED_WAVES_2)))

template <class E, bool kGrouped, bool kNt, int kB, bool kWait>
__global__ __launch_bounds__(kBlock) DDL_FUSED_OCCUPANCY
void fused_kernel(RankPtrs bufs, FusedArgs a) {
    fused_body<E, kGrouped, kNt, false, false, kB, false, kWait>(bufs, a, nullptr);
}

template <class E, bool kGrouped, bool kNt, int kB>
__global__ __launch_bounds__(kBlock) DDL_FUSED_OCCUPANCY
void fused_sgd_kernel(RankPtrs bufs, FusedArgs a, SgdArgs g) {
    fused_body<E, kGrouped, kNt, true, false, kB>(bufs, a, &g);
}

// The reduce kernel of the two-kernel form, tile by tile: each workgroup
// reads its tile from all P ranks (loads in batches of kB ranks) and
// writes the result to the home buffer.
template <class E, bool kGrouped, bool kNt, int kB>
__global__ __launch_bounds__(kBlock) DDL_FUSED_OCCUPANCY
void fused_reduce_kernel(RankPtrs bufs, FusedArgs a) {
    fused_body<E, kGrouped, kNt, false, true, kB>(bufs, a, nullptr);
}

// The reduce kernel of the LARS step's two-kernel form: also the per-tile
// partial sums of the layer norms.
template <class E, bool kGrouped, bool kNt, int kB>
__global__ __launch_bounds__(kBlock) DDL_FUSED_OCCUPANCY
void fused_reduce_lars_kernel(RankPtrs bufs, FusedArgs a) {
    fused_body<E, kGrouped, kNt, false, true, kB, true>(bufs, a, nullptr);
}

// ---------------------------------------------------------------------------
// The reduce kernel of the two-kernel form, rank by rank.  Workgroup b takes
// the K consecutive tiles from tile_base + b K on (K = 6 from 32 ranks on,
// 4 below; each tile of any span: a tile's chain and bounds are its own)
// and walks the chain positions j = 0 .. P-1: at each, it loads the tiles'
// elements of their chain entry j, one vector per lane per tile, and adds
// them to the tiles' sums, kReduceIssue loads at a time ahead of their
// adds.  Every element still takes its adds in chain order (groups of
// `group` entries, then the group sums), so the results are the bits of
// the tile-by-tile walk.  Lanes past a tile's whole vectors re-load its
// last one; a tile's last elements (fewer than a vector, or all of a span
// whose offset is not vector-aligned) are summed one by one after the
// walk.  Measured on MI355X as plain kernels over the pass's own geometry
// (40 ranks, 18.75 MB slices of 1.2 GB buffers, the ring's chunks with
// anchored tiles, 8 tiles per workgroup): loads two at a time 123 us per
// bucket, four at a time 128, all eight 131, one 169; tile by tile with
// batches of 4 ranks 134.  In the pass, 6 tiles per workgroup (a third
// more workgroups per bucket) beat 8 by 1-1.5% per step.
// ---------------------------------------------------------------------------

// Zeros to load for a tile with no whole vectors (room for the widest
// vector loaded, eight binary32 weights).
__device__ __align__(32) const uint32_t kZeroVec[8] = {0, 0, 0, 0, 0, 0, 0, 0};

// M binary64 sums over the workgroup at once, each exactly as block_sum
// forms it (the same butterfly within each wave, then the waves' sums in
// wave order from zero), with one barrier.  The results are in v[] of
// lane 0 of wave 0; every lane of the workgroup must call it.
template <int M>
__device__ __forceinline__ void block_sums(double (&v)[M], double (*lds)[M]) {
#pragma unroll
    for (int j = 0; j < M; ++j)
#pragma unroll
        for (int o = 32; o > 0; o >>= 1)
            v[j] += __shfl_xor(v[j], o, 64);
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    if (lane == 0)
#pragma unroll
        for (int j = 0; j < M; ++j)
            lds[wave][j] = v[j];
    __syncthreads();
    if (threadIdx.x == 0)
#pragma unroll
        for (int j = 0; j < M; ++j) {
            double s = 0.0;
            for (int i = 0; i < kBlock / 64; ++i)
                s += lds[i][j];
            v[j] = s;
        }
}

template <class E, bool kGrouped, bool kNt, bool kLars, int K>
__device__ __forceinline__ void reduce_tiles(const RankPtrs &bufs, const FusedArgs &a) {
    using T = typename E::T;
    using V = typename E::V;
    using Wv = typename E::W;
    static_assert(fused_vecs_per_lane(sizeof(T)) == 1, "one vector per lane per tile");
    constexpr uint64_t kTile = fused_tile_elems(sizeof(T));
    constexpr int kIssue = kReduceIssue;
    static_assert(K % kIssue == 0, "loads in whole groups");
    constexpr int kZeroSlot = K;
    // rank addresses in chain order: one slot per distinct span of the
    // workgroup's tiles, and a slot whose every entry is the zero vector
    __shared__ uint64_t src[K + 1][DDL_MAX_RANKS];
    __shared__ double lds_norm[kLars ? kBlock / 64 : 1][2 * K];
    const int P = a.P;
    const uint32_t tid = threadIdx.x;
    const uint32_t first = a.tile_base + blockIdx.x * (uint32_t)K;
    const uint32_t nt = min((uint32_t)K, a.tile_end - first);
    uint64_t base[K];     // first element of each tile
    uint32_t cnt[K];      // its elements
    uint32_t nvec[K];     // its whole vectors (none when its span is not aligned)
    int slot[K];          // the slot of its span's chain
    uint32_t coff[K];     // chain offset of each slot
    int nslots = 0;
    uint32_t prev = UINT32_MAX;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        base[k] = 0;
        cnt[k] = nvec[k] = 0;
        slot[k] = kZeroSlot;
        coff[k] = 0;
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if ((uint32_t)k < nt) {
            const uint32_t tile = first + (uint32_t)k;
            const uint32_t i = a.tile_span[tile];
            const DevSpan sp = a.spans[i];
            const uint64_t j = tile - a.prefix[i];
            const uint64_t sh = tile_shift(sp.off, kTile, a.anchor);
            base[k] = tile_lo(sp.off, sh, kTile, j);
            cnt[k] = (uint32_t)(tile_hi(sp.off, sp.len, sh, kTile, j) - base[k]);
            nvec[k] = (sp.flags & kItemAligned) ? cnt[k] / E::N : 0;
            // consecutive tiles of one span are adjacent
            if (i != prev) {
#pragma unroll
                for (int q = 0; q < K; ++q)
                    if (q == nslots)
                        coff[q] = sp.chain_off;
                ++nslots;
                prev = i;
            }
            slot[k] = nslots - 1;
        }
    }
    // every slot's entries at once: one dependent pair of loads per lane
    for (int m = (int)tid; m < (nslots + 1) * P; m += kBlock) {
        const int q = m / P, r = m - q * P;
        uint64_t addr = reinterpret_cast<uint64_t>(&kZeroVec);
        if (q < nslots) {
            uint32_t co = coff[0];
#pragma unroll
            for (int q2 = 1; q2 < K; ++q2)
                if (q == q2)
                    co = coff[q2];
            addr = reinterpret_cast<uint64_t>(bufs.p[a.chains[co + r]]);
        }
        src[q < nslots ? q : kZeroSlot][r] = addr;
    }
    // Every load of the walk is unconditional (branches around them would
    // keep K values live per path): lanes past a tile's whole vectors
    // re-load its last one (a line already in flight), and a tile without
    // whole vectors (or past the launch's last tile) reads the zero vector
    // at every chain position.
    int vslot[K];
    uint64_t lane_off[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        vslot[k] = nvec[k] ? slot[k] : kZeroSlot;
        lane_off[k] = nvec[k] ? (base[k] + (uint64_t)min(tid, nvec[k] - 1) * E::N) * sizeof(T)
                              : 0;
    }
    __syncthreads();
    Chain<E> c[K];
    V acc[K];
    for (int r = 0; r < P; ++r) {
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += kIssue) {
            V x[kIssue];
#pragma unroll
            for (int q = 0; q < kIssue; ++q)
                x[q] = ld_global<V, kNt>(src[vslot[k0 + q]][r] + lane_off[k0 + q]);
            // the group's loads issue before its adds: left alone, the
            // scheduler may keep a single load in flight
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < kIssue; ++q) {
                const int k = k0 + q;
                if (kGrouped)
                    c[k].push(x[q], a.group);
                else
                    acc[k] = r == 0 ? x[q] : E::add(acc[k], x[q]);
            }
        }
    }
    // kLars: replica 0's weights of the tiles' vectors, loaded before the
    // results are stored (replicas never overlap the gradient buffers)
    Wv wv[kLars ? K : 1];
    if constexpr (kLars)
#pragma unroll
        for (int k = 0; k < K; ++k)
            wv[k] = ld_stream<Wv, true>(
                nvec[k] ? static_cast<const void *>(a.w0 + base[k] +
                                                    (uint64_t)min(tid, nvec[k] - 1) * E::N)
                        : static_cast<const void *>(kZeroVec));
#pragma unroll
    for (int k = 0; k < K; ++k) {
        V y = kGrouped ? c[k].acc : acc[k];
        if (a.mean)
            y = E::div(y, a.divisor);
        acc[k] = y;
        if (tid < nvec[k]) {
            const V one[1] = {y};
            store_home<E, 1>(a.home, base[k] + (uint64_t)tid * E::N, one);
        }
    }
    // each tile's last elements one by one, and (kLars) its norm partial
    // sums: each lane its vector, then its elements, then the workgroup
    double sums[kLars ? 2 * K : 1];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        double sw = 0.0, sy = 0.0;
        if ((uint32_t)k >= nt) {
            if constexpr (kLars)
                sums[2 * k] = sums[2 * k + 1] = 0.0;
            continue;
        }
        if constexpr (kLars) {
            if (tid < nvec[k]) {
                add_squares<Wv>(E::widen(acc[k]), sy);
                add_squares<Wv>(wv[k], sw);
            }
        }
        for (uint32_t m = nvec[k] * E::N + tid; m < cnt[k]; m += kBlock) {
            const uint64_t e = base[k] + m;
            T s = 0, gs = 0;
            int pos = 0;
            bool first_group = true;
            for (int j = 0; j < P; ++j) {
                const T v =
                    *reinterpret_cast<const T DDL_GLOBAL *>(src[slot[k]][j] + e * sizeof(T));
                gs = pos == 0 ? v : E::add1(gs, v);
                if (++pos == a.group) {
                    s = first_group ? gs : E::add1(s, gs);
                    first_group = false;
                    pos = 0;
                }
            }
            if (a.mean)
                s = E::div1(s, a.divisor);
            static_cast<T *>(a.home)[e] = s;
            if (kLars) {
                const double y = (double)(float)s, w = (double)a.w0[e];
                sy += y * y;
                sw += w * w;
            }
        }
        if constexpr (kLars) {
            sums[2 * k] = sw;
            sums[2 * k + 1] = sy;
        }
    }
    if constexpr (kLars) {
        block_sums<2 * K>(sums, lds_norm);
        if (tid == 0)
#pragma unroll
            for (int k = 0; k < K; ++k)
                if ((uint32_t)k < nt) {
                    a.partial[2 * (uint64_t)(first + k)] = sums[2 * k];
                    a.partial[2 * (uint64_t)(first + k) + 1] = sums[2 * k + 1];
                }
    }
}

template <class E, bool kGrouped, bool kNt, int K>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4)))
void fused_reduce_ranks_kernel(RankPtrs bufs, FusedArgs a) {
    reduce_tiles<E, kGrouped, kNt, false, K>(bufs, a);
}

// The same with the LARS step's per-tile partial sums of the layer norms.
template <class E, bool kGrouped, bool kNt, int K>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4)))
void fused_reduce_ranks_lars_kernel(RankPtrs bufs, FusedArgs a) {
    reduce_tiles<E, kGrouped, kNt, true, K>(bufs, a);
}

// ---------------------------------------------------------------------------
// broadcast: the second kernel of the two-kernel form.  Workgroup b copies
// tiles_per_group anchored tiles from tile (b / ngroups) * tiles_per_group
// on -- of the run [off, off + len), or of the bucket table -- from rank 0
// to ranks 1 + g * ranks_per_group ... (at most P - 1), g = b % ngroups.
// The copy is of the bits: no arithmetic.  In run mode no table is read, so
// a workgroup's first access is the load of the values it copies.
// ---------------------------------------------------------------------------
// One tile of the broadcast: tile q of the run (or table tile q past
// tile_base) to ranks r0 .. r1.  kUpd (table mode, the LARS step): with the
// reduced values in hand, also step the weight replicas of rank group grp
// (see BcastArgs) by the tile's bucket's rate.
template <class E, bool kUpd, int kRB = 1, bool kWait = false>
__device__ __forceinline__ void bcast_tile(const RankPtrs &bufs, const BcastArgs &a, uint64_t q,
                                           int r0, int r1, const RankPtrs *w, uint32_t grp) {
    using T = typename E::T;
    using V = typename E::V;
    using Wv = typename E::W;
    constexpr int U = fused_vecs_per_lane(sizeof(T));
    constexpr uint64_t kTile = fused_tile_elems(sizeof(T));
    constexpr uint64_t kStride = (uint64_t)kBlock * E::N;
    const uint32_t tid = threadIdx.x;
    uint64_t off = a.off, len = a.len, j = q;
    bool aligned = a.aligned != 0;
    uint32_t bucket = 0;
    if (a.spans) {
        if (q >= (uint64_t)(a.tile_end - a.tile_base))
            return;
        const uint32_t tile = a.tile_base + (uint32_t)q;
        bucket = a.tile_span[tile];
        const DevSpan sp = a.spans[bucket];
        off = sp.off;
        len = sp.len;
        aligned = (sp.flags & kItemAligned) != 0;
        j = tile - a.prefix[bucket];
    }
    const uint64_t sh = tile_shift(off, kTile, true);
    if (j >= tile_count(len, sh, kTile))
        return;
    const uint64_t base = tile_lo(off, sh, kTile, j);
    const uint32_t cnt = (uint32_t)(tile_hi(off, len, sh, kTile, j) - base);
    const T DDL_GLOBAL *home =
        reinterpret_cast<const T DDL_GLOBAL *>(reinterpret_cast<uint64_t>(bufs.p[0]));
    // the replicas this workgroup steps: replica 0 for the first rank group
    // (k = -1; no rank group writes rank 0), then replicas w0 .. w1 - 1 (its
    // own ranks, with one replica per rank)
    const bool rep0 = kUpd && grp == 0;
    const int w0 = kUpd && a.nweights > 1 ? r0 : 0, w1 = kUpd && a.nweights > 1 ? r1 : 0;
    const float rate = kUpd ? (a.rate ? a.rate[bucket] : a.lr) : 0.0f;
    uint32_t done = 0;
    if (aligned) {
        const uint32_t nvec = cnt / E::N;
        if (nvec == (uint32_t)(U * kBlock)) {
            const uint64_t e = base + (uint64_t)tid * E::N;
            V v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = *reinterpret_cast<const V DDL_GLOBAL *>(home + e + u * kStride);
            for (int r = r0; r < r1; ++r) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    st_stream<V>(static_cast<T *>(bufs.p[r]) + e + u * kStride, v[u]);
                if (kWait)
                    wait_stores();
            }
            if (kUpd) {
                // replicas in batches of kRB: every load of a batch is issued
                // before its stores (a wave keeps kRB requests in flight)
                const int nrep = (rep0 ? 1 : 0) + (w1 - w0);
                for (int j0 = 0; j0 < nrep; j0 += kRB) {
                    Wv x[kRB][U];
#pragma unroll
                    for (int k = 0; k < kRB; ++k)
                        if (j0 + k < nrep) {
                            const int j = j0 + k;
                            const int r = rep0 ? (j == 0 ? 0 : w0 + j - 1) : w0 + j;
                            const float *wr = static_cast<const float *>(w->p[r]) + e;
#pragma unroll
                            for (int u = 0; u < U; ++u)
                                x[k][u] = ld_stream<Wv, true>(wr + u * kStride);
                        }
#pragma unroll
                    for (int k = 0; k < kRB; ++k)
                        if (j0 + k < nrep) {
                            const int j = j0 + k;
                            const int r = rep0 ? (j == 0 ? 0 : w0 + j - 1) : w0 + j;
                            float *wr = static_cast<float *>(w->p[r]) + e;
#pragma unroll
                            for (int u = 0; u < U; ++u)
                                st_stream<Wv>(wr + u * kStride,
                                              sgd_step<Wv>(x[k][u], E::widen(v[u]), rate));
                        }
                    if (kWait)
                        wait_stores();
                }
            }
        } else {
            for (uint32_t k = tid; k < nvec; k += kBlock) {
                const uint64_t e = base + (uint64_t)k * E::N;
                const V v = *reinterpret_cast<const V DDL_GLOBAL *>(home + e);
                for (int r = r0; r < r1; ++r)
                    st_stream<V>(static_cast<T *>(bufs.p[r]) + e, v);
                if (kUpd)
                    for (int k = rep0 ? -1 : 0; k < w1 - w0; ++k) {
                        float *wr = static_cast<float *>(w->p[k < 0 ? 0 : w0 + k]) + e;
                        st_stream<Wv>(wr, sgd_step<Wv>(ld_stream<Wv, true>(wr), E::widen(v),
                                                       rate));
                    }
            }
        }
        done = nvec * E::N;
    }
    for (uint32_t k = done + tid; k < cnt; k += kBlock) {
        const uint64_t e = base + k;
        const T x = home[e];
        for (int r = r0; r < r1; ++r)
            static_cast<T *>(bufs.p[r])[e] = x;
        if (kUpd)
            for (int k = rep0 ? -1 : 0; k < w1 - w0; ++k) {
                float *wr = static_cast<float *>(w->p[k < 0 ? 0 : w0 + k]) + e;
                *wr = sgd_step<float>(*wr, (float)x, rate);
            }
    }
}

// Workgroup b: rank group g = b % ngroups, tiles (b / ngroups) * tpg ...
// + tpg - 1 (tpg = tiles_per_group).  With nxcd > 1 the workgroups are
// dealt so that all rank groups of a tile block run on one accelerator die
// (workgroup b runs on die b % nxcd), which then fetches the block's values
// into its L2 once instead of once per die.
template <class E, bool kUpd, int kRB = 1, bool kWait = false>
__device__ __forceinline__ void bcast_body(const RankPtrs &bufs, const BcastArgs &a,
                                           const RankPtrs *w) {
    const uint32_t ng = (uint32_t)a.ngroups;
    uint32_t qb, grp;
    if (a.nxcd > 1) {
        const uint32_t x = blockIdx.x % (uint32_t)a.nxcd, jj = blockIdx.x / (uint32_t)a.nxcd;
        qb = x + (uint32_t)a.nxcd * (jj / ng);
        grp = jj % ng;
    } else {
        qb = blockIdx.x / ng;
        grp = blockIdx.x % ng;
    }
    const int r0 = 1 + (int)grp * a.ranks_per_group;
    const int r1 = min(a.P, r0 + a.ranks_per_group);
    const uint64_t q0 = (uint64_t)qb * (uint64_t)a.tiles_per_group;
    for (int k = 0; k < a.tiles_per_group; ++k)
        bcast_tile<E, kUpd, kRB, kWait>(bufs, a, q0 + (uint64_t)k, r0, r1, w, grp);
}

template <class E, bool kWait>
__global__ __launch_bounds__(kBlock) void bcast_kernel(RankPtrs bufs, BcastArgs a) {
    bcast_body<E, false, 1, kWait>(bufs, a, nullptr);
}

// The broadcast of the two-kernel form with the update of the weight
// replicas w riding on it: the LARS step (each bucket's rate) or the SGD
// step with kept gradients (the constant rate lr), kRB replicas' loads ahead
// of their stores (knob DDL_TUNE_UPDATE_BATCH, as the update kernel).
template <class E, int kRB, bool kWait>
__global__ __launch_bounds__(kBlock) void bcast_update_kernel(RankPtrs bufs, RankPtrs w,
                                                              BcastArgs a) {
    bcast_body<E, true, kRB, kWait>(bufs, a, &w);
}

// ---------------------------------------------------------------------------
// tiny spans: a group made only of spans of at most kTinySpanMax elements.
// Wave w of workgroup b takes tiny span lo + 4 b + w, lane l its element l:
// the chain is walked in the span's order (groups of `group` entries, then
// the group sums), the mean applied, and the result written to every rank,
// exactly as the one-kernel pass does.  Loads go out kTinyBatch at a time
// ahead of their adds.  No barrier: whole waves and lanes may leave early.
// ---------------------------------------------------------------------------
constexpr int kTinyBatch = 8;

template <class E>
__global__ __launch_bounds__(kBlock) void tiny_kernel(RankPtrs bufs, TinyArgs a) {
    using T = typename E::T;
    const uint32_t t = a.lo + blockIdx.x * (uint32_t)(kBlock / 64) + (threadIdx.x >> 6);
    if (t >= a.hi)
        return;
    const DevSpan sp = a.spans[a.tiny[t]];
    const uint32_t lane = threadIdx.x & 63u;
    if (lane >= sp.len)
        return;
    const uint64_t e = sp.off + lane;
    const uint8_t *ch = a.chains + sp.chain_off;
    const int P = a.P;
    T acc = 0, gacc = 0;
    int pos = 0;
    bool first_group = true;
    for (int b = 0; b < P; b += kTinyBatch) {
        T x[kTinyBatch];
#pragma unroll
        for (int j = 0; j < kTinyBatch; ++j)
            if (b + j < P)
                x[j] = *(reinterpret_cast<const T DDL_GLOBAL *>(
                             reinterpret_cast<uint64_t>(bufs.p[ch[b + j]])) + e);
#pragma unroll
        for (int j = 0; j < kTinyBatch; ++j)
            if (b + j < P) {
                gacc = pos == 0 ? x[j] : E::add1(gacc, x[j]);
                if (++pos == a.group) {
                    acc = first_group ? gacc : E::add1(acc, gacc);
                    first_group = false;
                    pos = 0;
                }
            }
    }
    if (a.mean)
        acc = E::div1(acc, a.divisor);
    for (int r = 0; r < P; ++r)
        static_cast<T *>(bufs.p[r])[e] = acc;
}

}  // namespace

namespace {

// One-kernel pass (home false; with the SGD step when sgd is set) or reduce
// kernel (home true) with kB loads per batch.
// Whether the one-kernel pass waits for each rank's stores to complete
// before storing to the next (DDL_TUNE_FUSED_STORE_WAIT: 0 never, 1 always,
// otherwise for binary32 groups of at least 2^27 elements per rank from 8
// ranks on).  Measured on MI355X, paired in one process: 8 ranks 300M
// elements -1.7..-3.3% (a 4-ring multi-ring -4.7%), 200M -1.7%, 128M
// -0.3%; 16 ranks 150M -0.3%; 4 ranks +2.0..+2.7%; smaller groups -0.1..
// +4.4% (8-40 ranks, 8M-64M elements); binary16 +0.7% at 8 ranks 300M.
bool fused_store_wait(const FusedArgs &a, size_t esize) {
    const int k = tuning(DDL_TUNE_FUSED_STORE_WAIT);
    if (k == 0 || k == 1)
        return k == 1;
    const uint64_t elems = (uint64_t)(a.tile_end - a.tile_base) * fused_tile_elems(esize);
    return esize == 4 && a.P >= 8 && elems >= (1ull << 27);
}

template <class E, bool kGrouped, bool kNt, int kB>
void launch_b(dim3 grid, hipStream_t s, const RankPtrs &bufs, const FusedArgs &a,
              const SgdArgs *sgd, bool home) {
    const dim3 block(kBlock);
    if (home && a.partial)
        hipLaunchKernelGGL((fused_reduce_lars_kernel<E, kGrouped, kNt, kB>), grid, block, 0, s,
                           bufs, a);
    else if (home)
        hipLaunchKernelGGL((fused_reduce_kernel<E, kGrouped, kNt, kB>), grid, block, 0, s, bufs,
                           a);
    else if (sgd)
        hipLaunchKernelGGL((fused_sgd_kernel<E, kGrouped, kNt, kB>), grid, block, 0, s, bufs, a,
                           *sgd);
    else if (fused_store_wait(a, sizeof(typename E::T)))
        hipLaunchKernelGGL((fused_kernel<E, kGrouped, kNt, kB, true>), grid, block, 0, s, bufs,
                           a);
    else
        hipLaunchKernelGGL((fused_kernel<E, kGrouped, kNt, kB, false>), grid, block, 0, s, bufs,
                           a);
}

template <class E, bool kGrouped, bool kNt>
void launch_nt(dim3 grid, hipStream_t s, const RankPtrs &bufs, const FusedArgs &a,
               const SgdArgs *sgd, bool home, int batch) {
    switch (batch) {
    case 2: launch_b<E, kGrouped, kNt, 2>(grid, s, bufs, a, sgd, home); break;
    case 4: launch_b<E, kGrouped, kNt, 4>(grid, s, bufs, a, sgd, home); break;
    case 8: launch_b<E, kGrouped, kNt, 8>(grid, s, bufs, a, sgd, home); break;
    default: launch_b<E, kGrouped, kNt, 1>(grid, s, bufs, a, sgd, home); break;
    }
}

// The rank-by-rank reduce kernel (with the LARS partial sums when
// a.partial is set).
template <class E, bool kGrouped, bool kNt, int K>
void launch_ranks_k(dim3 grid, hipStream_t s, const RankPtrs &bufs, const FusedArgs &a) {
    const dim3 block(kBlock);
    if (a.partial)
        hipLaunchKernelGGL((fused_reduce_ranks_lars_kernel<E, kGrouped, kNt, K>), grid, block, 0,
                           s, bufs, a);
    else
        hipLaunchKernelGGL((fused_reduce_ranks_kernel<E, kGrouped, kNt, K>), grid, block, 0, s,
                           bufs, a);
}

template <class E, bool kGrouped, bool kNt>
void launch_ranks(dim3 grid, hipStream_t s, const RankPtrs &bufs, const FusedArgs &a) {
    if (reduce_tiles_per_group(a.P) == kReduceTilesWide)
        launch_ranks_k<E, kGrouped, kNt, kReduceTilesWide>(grid, s, bufs, a);
    else
        launch_ranks_k<E, kGrouped, kNt, kReduceTilesNarrow>(grid, s, bufs, a);
}

template <class E, bool kGrouped>
void launch_e(dim3 grid, hipStream_t s, const RankPtrs &bufs, const FusedArgs &a,
              const SgdArgs *sgd, bool home, bool ranks) {
    if (home) {
        // the reduce kernel reads the ranks with non-temporal loads whatever
        // P: the P input streams must not evict the results the broadcast
        // kernel re-reads (measured on MI355X, 40 ranks: 6031 GB/s against
        // 5242 with cached loads)
        const bool nt = tuning(DDL_TUNE_REDUCE_NT_LOAD) != 0;
        if (ranks) {
            if (nt)
                launch_ranks<E, kGrouped, true>(grid, s, bufs, a);
            else
                launch_ranks<E, kGrouped, false>(grid, s, bufs, a);
            return;
        }
        const int batch = tuning(DDL_TUNE_REDUCE_BATCH);
        if (nt)
            launch_nt<E, kGrouped, true>(grid, s, bufs, a, nullptr, true, batch);
        else
            launch_nt<E, kGrouped, false>(grid, s, bufs, a, nullptr, true, batch);
        return;
    }
    constexpr int kLaneElems = fused_vecs_per_lane(sizeof(typename E::T)) * E::N;
    const bool nt = a.P * kLaneElems <= 4 * tuning(DDL_TUNE_FUSED_NT_LOAD_MAX_P);
    const int batch = tuning(DDL_TUNE_FUSED_BATCH);
    if (nt)
        launch_nt<E, kGrouped, true>(grid, s, bufs, a, sgd, false, batch);
    else
        launch_nt<E, kGrouped, false>(grid, s, bufs, a, sgd, false, batch);
}

}  // namespace

int launch_fused(int dtype, const RankPtrs &bufs, const FusedArgs &a, const SgdArgs *sgd,
                 bool home, uint32_t tiles, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the reduce kernel walks its workgroups' tiles rank by rank from
    // DDL_TUNE_REDUCE_RANKS_MIN_P ranks on, tile by tile below
    const bool ranks = home && a.P >= tuning(DDL_TUNE_REDUCE_RANKS_MIN_P);
    const uint32_t per =
        ranks ? (uint32_t)reduce_tiles_per_group(a.P) : (uint32_t)kFusedTilesPerGroup;
    dim3 grid((tiles + per - 1) / per);
    const bool grouped = a.group != a.P;
    if (dtype == DDL_F32) {
        if (grouped)
            launch_e<F32, true>(grid, s, bufs, a, sgd, home, ranks);
        else
            launch_e<F32, false>(grid, s, bufs, a, sgd, home, ranks);
    } else {
        if (grouped)
            launch_e<F16, true>(grid, s, bufs, a, sgd, home, ranks);
        else
            launch_e<F16, false>(grid, s, bufs, a, sgd, home, ranks);
    }
    return (int)hipGetLastError();
}

int launch_tiny(int dtype, const RankPtrs &bufs, const TinyArgs &a, void *stream) {
    if (a.hi <= a.lo)
        return (int)hipSuccess;
    constexpr uint32_t kWaves = kBlock / 64;
    const dim3 grid((a.hi - a.lo + kWaves - 1) / kWaves), block(kBlock);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == DDL_F32)
        hipLaunchKernelGGL((tiny_kernel<F32>), grid, block, 0, s, bufs, a);
    else
        hipLaunchKernelGGL((tiny_kernel<F16>), grid, block, 0, s, bufs, a);
    return (int)hipGetLastError();
}

namespace {

// Grid of a broadcast launch, or 0 with *bad set when it cannot be launched.
uint64_t bcast_blocks(int dtype, const BcastArgs &a, bool *bad) {
    const uint64_t tile = fused_tile_elems(dtype == DDL_F32 ? 4 : 2);
    const uint64_t tiles = a.spans ? (uint64_t)(a.tile_end - a.tile_base)
                                   : tile_count(a.len, tile_shift(a.off, tile, true), tile);
    *bad = a.ngroups < 1 || a.ranks_per_group < 1 || a.tiles_per_group < 1;
    if (*bad)
        return 0;
    const uint64_t qblocks = (tiles + (uint64_t)a.tiles_per_group - 1) / (uint64_t)a.tiles_per_group;
    const uint64_t blocks =
        a.nxcd > 1 ? (qblocks + (uint64_t)a.nxcd - 1) / (uint64_t)a.nxcd * (uint64_t)a.nxcd *
                         (uint64_t)a.ngroups
                   : qblocks * (uint64_t)a.ngroups;
    *bad = blocks * kBlock > 0xffffffffull;
    return *bad ? 0 : blocks;
}

template <class E, bool kWait>
void launch_bcast_update_t(int batch, dim3 grid, hipStream_t s, const RankPtrs &bufs,
                           const RankPtrs &w, const BcastArgs &a) {
    const dim3 block(kBlock);
    if (batch <= 1)
        hipLaunchKernelGGL((bcast_update_kernel<E, 1, kWait>), grid, block, 0, s, bufs, w, a);
    else if (batch == 2)
        hipLaunchKernelGGL((bcast_update_kernel<E, 2, kWait>), grid, block, 0, s, bufs, w, a);
    else
        hipLaunchKernelGGL((bcast_update_kernel<E, 4, kWait>), grid, block, 0, s, bufs, w, a);
}

template <bool kWait>
void launch_bcast_update_e(int dtype, int batch, dim3 grid, hipStream_t s, const RankPtrs &bufs,
                           const RankPtrs &w, const BcastArgs &a) {
    if (dtype == DDL_F32)
        launch_bcast_update_t<F32, kWait>(batch, grid, s, bufs, w, a);
    else
        launch_bcast_update_t<F16, kWait>(batch, grid, s, bufs, w, a);
}

// Whether the broadcast waits for each rank's stores to complete before
// storing to the next (DDL_TUNE_BCAST_STORE_WAIT: 0 never, 1 always,
// otherwise for binary32).  A wave that leaves right after issuing its
// stores lets the next workgroup's pile up behind them.  Measured on
// MI355X, paired in one process (two runs): the ResNet-50 multi-ring -2.1..
// -2.6% per pass, the 40-rank step -0.55% (all-reduce, SGD and LARS alike),
// a 16-rank ring -0.1%; binary16 within +-1% either way (the torus +1.6,
// +0.7, -0.4%, the multi-ring +1.0%).  In a plain probe kernel (one 4 KB
// tile to 2 ranks per workgroup) the wait took the broadcast from 152 to
// 120 us per 18.75 MB bucket.
bool bcast_store_wait(int dtype) {
    const int k = tuning(DDL_TUNE_BCAST_STORE_WAIT);
    return k == 0 ? false : k == 1 ? true : dtype == DDL_F32;
}

}  // namespace

int launch_bcast_update(int dtype, const RankPtrs &bufs, const RankPtrs &w, const BcastArgs &a,
                        void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    bool bad = false;
    const uint64_t blocks = bcast_blocks(dtype, a, &bad);
    if (bad || !a.spans || a.nweights < 1)
        return (int)hipErrorInvalidValue;
    if (blocks == 0)
        return (int)hipSuccess;
    const dim3 grid((uint32_t)blocks);
    const int batch = tuning(DDL_TUNE_UPDATE_BATCH);
    if (bcast_store_wait(dtype))
        launch_bcast_update_e<true>(dtype, batch, grid, s, bufs, w, a);
    else
        launch_bcast_update_e<false>(dtype, batch, grid, s, bufs, w, a);
    return (int)hipGetLastError();
}

int launch_bcast(int dtype, const RankPtrs &bufs, const BcastArgs &a, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint64_t tile = fused_tile_elems(dtype == DDL_F32 ? 4 : 2);
    const uint64_t tiles = a.spans ? (uint64_t)(a.tile_end - a.tile_base)
                                   : tile_count(a.len, tile_shift(a.off, tile, true), tile);
    if (a.ngroups < 1 || a.ranks_per_group < 1 || a.tiles_per_group < 1)
        return (int)hipErrorInvalidValue;
    const uint64_t qblocks = (tiles + (uint64_t)a.tiles_per_group - 1) / (uint64_t)a.tiles_per_group;
    const uint64_t blocks =
        a.nxcd > 1 ? (qblocks + (uint64_t)a.nxcd - 1) / (uint64_t)a.nxcd * (uint64_t)a.nxcd *
                         (uint64_t)a.ngroups
                   : qblocks * (uint64_t)a.ngroups;
    if (blocks * kBlock > 0xffffffffull)
        return (int)hipErrorInvalidValue;
    if (blocks == 0)
        return (int)hipSuccess;
    const dim3 grid((uint32_t)blocks), block(kBlock);
    const bool wait = bcast_store_wait(dtype);
    if (dtype == DDL_F32) {
        if (wait)
            hipLaunchKernelGGL((bcast_kernel<F32, true>), grid, block, 0, s, bufs, a);
        else
            hipLaunchKernelGGL((bcast_kernel<F32, false>), grid, block, 0, s, bufs, a);
    } else {
        if (wait)
            hipLaunchKernelGGL((bcast_kernel<F16, true>), grid, block, 0, s, bufs, a);
        else
            hipLaunchKernelGGL((bcast_kernel<F16, false>), grid, block, 0, s, bufs, a);
    }
    return (int)hipGetLastError();
}

}  // namespace ddl
