// ddl_internal.h -- layouts shared by the schedule generator (host C++) and
// the gfx950 kernels.  Not part of the public interface.
#pragma once

#include <stdint.h>

#include "../../include/ddl.h"

namespace ddl {

// One workgroup = 256 lanes = 4 wave64 (tuning knob).
#ifndef DDL_BLOCK
#define DDL_BLOCK 256
#endif
constexpr int kBlock = DDL_BLOCK;
// Every lane moves 16 bytes per vector access (one dwordx4).
constexpr int kVecBytes = 16;
// Vectors per lane per tile: step kernels (one source, one destination)
// and the fused kernel (P sources, P destinations).  Tuning knobs.
#ifndef DDL_FUSED_VPL_F32
#define DDL_FUSED_VPL_F32 1
#endif
#ifndef DDL_FUSED_VPL_F16
#define DDL_FUSED_VPL_F16 1
#endif
#ifndef DDL_FUSED_TPW
#define DDL_FUSED_TPW 1
#endif
// Fused pass, vectors per lane per tile: one dwordx4 of either type.
// Measured on MI355X (paired, three rounds), binary16 with one against two:
// 16-rank torus fused -2%, persistent stepwise -6%; 8-rank ring one kernel
// -4.5%; mixed-precision ResNet-50 stepwise -8.6%.  Binary32 with two or
// four: -3%, -8% at 40 ranks.
constexpr int fused_vecs_per_lane(int esz) {
    return esz == 4 ? DDL_FUSED_VPL_F32 : DDL_FUSED_VPL_F16;
}
// Consecutive tiles one fused workgroup walks (address translations of the
// P rank streams are reused from tile to tile).
constexpr int kFusedTilesPerGroup = DDL_FUSED_TPW;
// The two-kernel form's reduce kernel rank by rank (fused_kernel.hip,
// reduce_tiles): consecutive tiles one workgroup takes -- 6 from 32 ranks
// on, 4 below -- and the loads it issues at a time ahead of their adds.
// Measured on MI355X, paired against the reduce tile by tile: 40 ranks 8
// tiles -3.3% per pass (4: -1.5%), and 6 tiles a further -1.0..-1.5% per
// step against 8 (10 or 12: +7%, +15%); 16 ranks 4 tiles, the binary16
// torus -1.6..-2.2% and the multi-ring ResNet-50 -0.7% (6 tiles: the
// same within 1%; 8: +1.5..+3%); loads one or four at a time lose at both
// sizes.  The tile count must be a multiple of the load group.
#ifndef DDL_REDUCE_TILES_WIDE
#define DDL_REDUCE_TILES_WIDE 6
#endif
#ifndef DDL_REDUCE_TILES_NARROW
#define DDL_REDUCE_TILES_NARROW 4
#endif
#ifndef DDL_REDUCE_ISSUE
#define DDL_REDUCE_ISSUE 2
#endif
constexpr int kReduceTilesWide = DDL_REDUCE_TILES_WIDE;
constexpr int kReduceTilesNarrow = DDL_REDUCE_TILES_NARROW;
constexpr int kReduceIssue = DDL_REDUCE_ISSUE;
constexpr int reduce_tiles_per_group(int P) {
    return P >= 32 ? kReduceTilesWide : kReduceTilesNarrow;
}

// Elements of one tile, by element size.
// Step kernels take 1, 2 or 4 vectors per lane per tile; each plan picks
// one from the length of its items (schedule.cpp, pick_step_vpl).
constexpr uint64_t step_tile_elems(int esz, int vpl) {
    return (uint64_t)kBlock * vpl * (kVecBytes / esz);
}
constexpr uint64_t fused_tile_elems(int esz) {
    return (uint64_t)kBlock * fused_vecs_per_lane(esz) * (kVecBytes / esz);
}

// Tiling of a range [off, off + len): tile j covers
// [max(off, off - s + j * tile), min(off + len, off - s + (j + 1) * tile)).
// With s = off % tile ("anchored") every tile but the range's first and
// last starts at a multiple of the tile size (4 KB for the fused pass), so a
// wave's 1 KB access covers whole 128-byte cache lines; with s = 0 the tiles
// start at off.  Measured on MI355X, tiles starting 16-48 bytes into a line
// cost 9% (one-kernel pass) to 15% (two-kernel pass) at 40 ranks, and the
// schedule's chunk boundaries fall on 16-byte multiples only.  Anchoring
// costs a tile per range, so tables of short ranges keep s = 0.
constexpr uint64_t tile_shift(uint64_t off, uint64_t tile, bool anchor) {
    return anchor ? off % tile : 0;
}
constexpr uint64_t tile_count(uint64_t len, uint64_t s, uint64_t tile) {
    return len ? (s + len + tile - 1) / tile : 0;
}
constexpr uint64_t tile_lo(uint64_t off, uint64_t s, uint64_t tile, uint64_t j) {
    return j == 0 ? off : off - s + j * tile;
}
constexpr uint64_t tile_hi(uint64_t off, uint64_t len, uint64_t s, uint64_t tile, uint64_t j) {
    return off - s + (j + 1) * tile < off + len ? off - s + (j + 1) * tile : off + len;
}

enum : uint32_t {
    kItemDivide = 1u,   // divide by P after the add (mean epilogue)
    kItemAligned = 2u,  // offset is a multiple of 16 B / element size
    kItemFinal = 4u,    // this add completes the chunk's sum (its owner)
};

// One pair transfer of one step (device layout, 32 bytes).
struct DevItem {
    uint64_t off;    // first element
    uint64_t len;    // elements
    int32_t src;     // sending rank
    int32_t dst;     // receiving rank
    uint32_t flags;  // kItem*
    uint32_t pad;
};

// One span of the fused pass (device layout, 24 bytes): elements
// [off, off+len) are summed over chain[chain_off .. chain_off+P).
struct DevSpan {
    uint64_t off;
    uint64_t len;
    uint32_t chain_off;
    uint32_t flags;  // kItemAligned
};

// Rank base pointers, passed by value as a kernel argument.
struct RankPtrs {
    void *p[DDL_MAX_RANKS];
};

// Arguments of one step launch: the tiles of items [item_lo, item_hi) of a
// step; tile t of the launch is global tile prefix[item_lo] + t.
struct StepArgs {
    const DevItem *items;
    const uint32_t *prefix;
    uint32_t item_lo, item_hi;
    uint32_t tile_base;
    float divisor;   // P, for the mean
    int anchor;      // tiles anchored at multiples of the tile size
};

// Arguments of one fused launch over spans [span_lo, span_hi).
struct FusedArgs {
    const DevSpan *spans;
    const uint32_t *prefix;
    const uint32_t *tile_span;  // [t] span of tile t
    const uint8_t *chains;
    uint32_t span_lo, span_hi;
    uint32_t tile_base;  // first tile of this launch
    uint32_t tile_end;   // one past the last tile of this launch
    int P;
    int group;       // chain entries per group (P for rings, cols for the torus)
    int mean;        // divide by P at the end
    float divisor;
    int anchor;      // tiles anchored at multiples of the tile size
    void *home;      // reduce kernel: where the result goes (rank 0's buffer,
                     // or a scratch buffer of n elements)
    // reduce kernel of the LARS step (null otherwise): per tile t of this
    // table, partial[2t] and partial[2t+1] receive the binary64 sums of
    // w0^2 and y^2 over the tile (w0 replica 0's binary32 weights)
    double *partial;
    const float *w0;
};

// Spans of at most kTinySpanMax elements are "tiny": a group made only of
// them (the BatchNorm and bias tensors of a ResNet, split over rings and
// ranks into pieces of a few elements) runs one wave per span, one element
// per lane, instead of one workgroup per span.
constexpr uint32_t kTinySpanMax = 64;
struct TinyArgs {
    const DevSpan *spans;
    const uint32_t *tiny;  // span indices of the tiny spans, in span order
    const uint8_t *chains;
    uint32_t lo, hi;       // entries [lo, hi) of tiny
    int P;
    int group;             // chain entries per group (as FusedArgs)
    int mean;
    float divisor;
};

// Arguments of one broadcast launch (second kernel of the two-kernel fused
// form): rank 0's values are copied to ranks 1..P-1, ranks_per_group of
// them per workgroup, so each tile of fused_tile_elems elements takes
// ngroups = ceil((P-1) / ranks_per_group) workgroups.  Two modes:
//  - run (spans == nullptr): the elements [off, off + len), one contiguous
//    run of memory; no table is read.  aligned: off is a multiple of 16 B.
//  - table: the anchored tiles [tile_base, tile_end) of the bucket table
//    spans / prefix / tile_span, for groups whose buckets are not one run.
struct BcastArgs {
    uint64_t off, len;
    const DevSpan *spans;
    const uint32_t *prefix;
    const uint32_t *tile_span;
    uint32_t tile_base, tile_end;
    int P;
    int ranks_per_group;
    int ngroups;
    int aligned;
    int tiles_per_group;  // consecutive tiles one workgroup copies
    int nxcd;             // > 1: all rank groups of a tile block on one die
    // the weight update riding on the broadcast (launch_bcast_update, table
    // mode): with the reduced values in hand, the workgroup of rank group g
    // also steps weight replicas -- those of its own ranks when nweights ==
    // P, plus replica 0 for g == 0; replica 0 alone for g == 0 when nweights
    // == 1 -- by w = w - rate[bucket] * y (the LARS step), or w = w - lr * y
    // when rate is null (the SGD step)
    const float *rate;
    float lr;
    int nweights;
};

// The SGD step fused into the all-reduce's epilogue: binary32 weight
// replicas w[0..nweights) (nweights 1 = one replica shared by all ranks,
// or P = one per rank) take w - lr * y once the reduced value y reaches
// them.  keep_grads = 0 (fused pass only) leaves the gradient buffers as
// they were instead of writing y back.
struct SgdArgs {
    RankPtrs w;
    float lr;
    int nweights;
    int keep_grads;
};

// The LARS step after the all-reduce, layer = bucket (lars_kernels.hip):
// per-tile binary64 sums of squares, per-bucket rates, then the SGD step of
// every replica with its bucket's rate.  The tiles are the buckets' anchored
// tiles of fused_tile_elems elements (Schedule::bk_spans, bk_prefix,
// bk_of_tile).
struct LarsArgs {
    const DevSpan *spans;          // one per bucket
    const uint32_t *prefix;        // [i] first tile of bucket i, nbuckets + 1
    const uint32_t *tile_span;     // [t] bucket of tile t
    const void *y;                 // the reduced gradient: rank 0's buffer
    uint32_t tile_base, tile_end;  // norm and update launches: these tiles
    uint32_t bucket_lo, bucket_hi; // rate launch: these buckets
    double *partial;               // [2t], [2t+1]: sums of w_0^2 and y^2 over tile t
    float *rate;                   // [i] the rate of bucket i; null: lr for all
                                   // (the plain SGD step)
    float *rate_out;               // null, or the caller's copy of rate
    float lr;
    int nweights;
    int reps_per_group;            // update: replicas each workgroup steps
    int ngroups;                   // update: workgroups per tile
    double coeff, eps;
};

// The allocation-free LARS entry point keeps its partial sums and rates in
// a fixed per-device scratch of this size: up to 512Ki tiles of partial sums
// over the plan's buckets (8 MiB; 536,870,912 binary32 elements in whole
// tiles) after which the rates
// start at a 256-byte boundary, up to 64Ki buckets (256 KiB).
constexpr size_t kLarsScratchPartialBytes = 8u << 20;
constexpr size_t kLarsScratchBytes = kLarsScratchPartialBytes + (256u << 10);
// The device address and size of that scratch on `device` (looked up once
// per device with the device current).  Returns a hipError_t.
int lars_scratch(int device, void **ptr, size_t *bytes);

// Current value of a ddl_tune_knob (its default unless ddl_set_tuning set it).
int tuning(int knob);

// Kernel launchers.  sgd may be null (plain all-reduce).  Return hipError_t.
int launch_step(int dtype, int kind, int vpl, const RankPtrs &bufs, const StepArgs &a,
                const SgdArgs *sgd, uint32_t tiles, void *stream);
// home: the reduce kernel of the two-kernel form (result to rank 0 only).
int launch_fused(int dtype, const RankPtrs &bufs, const FusedArgs &a, const SgdArgs *sgd,
                 bool home, uint32_t tiles, void *stream);
int launch_bcast(int dtype, const RankPtrs &bufs, const BcastArgs &a, void *stream);
// The broadcast with the update of the replicas w riding on it (the LARS
// step's rates, or the SGD step's constant lr when a.rate is null).
int launch_bcast_update(int dtype, const RankPtrs &bufs, const RankPtrs &w, const BcastArgs &a,
                        void *stream);
int launch_tiny(int dtype, const RankPtrs &bufs, const TinyArgs &a, void *stream);
// The persistent step kernel: tiles [a.tile_base, a.tile_base + tiles) of the
// fused span table, every schedule step walked by the workgroup of a tile
// (with sgd, the SGD step of each rank where the reduced value reaches it).
int launch_walk(int dtype, const RankPtrs &bufs, const FusedArgs &a, const SgdArgs *sgd,
                uint32_t tiles, void *stream);
// kind: DDL_K_LARS_NORM or DDL_K_UPDATE (blocks = tiles from
// a.tile_base), DDL_K_LARS_RATE (blocks = buckets from a.bucket_lo).
int launch_lars(int dtype, int kind, const RankPtrs &w, const LarsArgs &a, uint32_t blocks,
                void *stream);

}  // namespace ddl
