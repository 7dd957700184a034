// step_kernels.hip -- one launch per schedule step (gfx950).
//
// A launch covers every pair of every ring of every bucket in the group: the
// schedule is race-free within a step, so all pairs run at once.  Each lane
// moves dwordx4 vectors of one source and one destination chunk.  The
// stores stay cached: the next step reads what this one wrote.
#include "device_common.h"

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
