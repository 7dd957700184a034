// schedule.h -- host schedule generator: turns (P, n, topology, buckets)
// into the step tables and fused-span tables the kernels walk.
#pragma once

#include <stdint.h>

#include <vector>

#include "ddl_internal.h"

namespace ddl {

struct Bucket {
    uint64_t off, len;
};

struct Schedule {
    // arguments
    int P = 0;
    uint64_t n = 0;
    int dtype = DDL_F32;
    int esz = 4;
    uint64_t q = 4;          // split quantum: 16 bytes / element size
    int op = DDL_SUM;
    int kind = DDL_RING;
    int k = 1;               // rings (multi-ring), 1 otherwise
    int rows = 1, cols = 1;  // torus grid
    std::vector<int> order;  // k*P: ring j puts rank order[j*P + x] at position x
    std::vector<Bucket> buckets;  // issue order

    // step tables.  Step s of every bucket forms one list, bucket-major, so
    // any run of consecutive buckets is a contiguous item range of a step.
    int nsteps = 0;
    std::vector<int> step_kind;                  // [s] DDL_K_REDUCE | DDL_K_GATHER
    std::vector<std::vector<DevItem>> items;     // [s] items
    std::vector<std::vector<uint32_t>> item_at;  // [s] first item of bucket b, nb+1
    std::vector<std::vector<uint32_t>> prefix;   // [s] tile prefix, nitems+1
    int step_vpl = 4;                            // step kernels' vectors per lane
    bool step_anchor = false;                    // step tiles anchored (ddl_internal.h)

    // fused tables: spans bucket-major, P chain entries each
    int group = 1;                       // chain entries per group
    std::vector<DevSpan> spans;
    std::vector<uint32_t> span_at;       // first span of bucket b, nb+1
    std::vector<uint32_t> span_prefix;   // tile prefix, nspans+1
    std::vector<uint32_t> span_of_tile;  // [t] the span fused tile t belongs to
    bool fused_anchor = false;           // fused tiles anchored (ddl_internal.h)
    std::vector<uint32_t> tiny;          // spans of <= kTinySpanMax elements, in order
    std::vector<uint32_t> tiny_prefix;   // tiny spans before span i, nspans+1

    // broadcast tables (two-kernel fused form, groups whose buckets are not
    // one contiguous run): a DevSpan per bucket (chain unused), its anchored
    // fused-tile prefix, and the bucket of every such tile
    std::vector<DevSpan> bk_spans;
    std::vector<uint32_t> bk_prefix;
    std::vector<uint32_t> bk_of_tile;
    std::vector<uint8_t> chains;

    // accounting
    std::vector<uint64_t> sent;          // [P] elements sent per rank
    uint64_t step_bytes = 0;             // HBM bytes of the stepwise path
    uint64_t fused_bytes = 0;            // HBM bytes of the fused path
};

// Split of a length-L segment into m pieces with quantum q: piece c is
// [b[c], b[c+1]), b[c] = min(L, q*floor(c*ceil(L/q)/m)).
void split_segment(uint64_t L, int m, uint64_t q, std::vector<uint64_t> &b);

// Validates the arguments and builds every table.  Returns a DDL_* code.
// exact: the buckets must tile [0, n) exactly; otherwise (one element type
// of a plan with typed buckets) they must only be disjoint and in range.
int build_schedule(Schedule &s, int P, uint64_t n, int dtype, int op,
                   const ddl_topo &topo, const ddl_bucket *buckets, int nbuckets,
                   bool exact = true);

// Proves the tables race-free: within one step no element of any rank that
// one item writes is read or written by another item.  Returns true if so.
bool check_schedule(const Schedule &s);

}  // namespace ddl
