// plan.cpp -- the C ABI: plans, the plan cache, and the bucket dispatcher.
//
// The dispatcher issues buckets in list order -- output layer first, so the
// all-reduce of the gradients back-propagation finishes first can overlap the
// rest of it (Baidu Ring-Allreduce article, part 4, opening paragraphs).  A
// bucket with a ready event waits for it on a side stream of the plan;
// consecutive buckets whose events are equal (NULL included) share one group
// of launches, so a step of all of them is one kernel.  With no event at all
// the work goes on the caller's stream directly.  A plan with typed buckets
// holds one schedule per element type, and a group runs one pass (or step
// sequence) per type it holds.
#include <hip/hip_runtime_api.h>

#include <limits.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "ddl_internal.h"
#include "schedule.h"

using namespace ddl;

constexpr int kMaxSideStreams = 4;
// Events a plan makes when it binds, for the completion tracking of the
// first caller streams it is executed on.
constexpr int kSpareEvents = 8;
// Flags of the completion-tracking events.  The host only asks them whether
// the plan's launches have finished (before its tables are freed); no
// stream waits for them and the host reads nothing the launches wrote, so
// they skip the system-scope fence (a cache writeback and invalidate) that
// an event record performs by default.  Measured on MI355X (paired, three
// rounds): back-to-back calls of the binary16 torus 305.6-306.6 -> 304.2-
// 304.4 us; a build with no record at all gained 2.8 us per call.
constexpr unsigned kTrackEventFlags = hipEventDisableTiming | hipEventDisableSystemFence;

// process-wide tuning knobs (ddl_set_tuning), stored as value + 1 so that
// the zero-initialised array means "every knob at its default"
constexpr int kTuneDefault[] = {
    0,   // DDL_TUNE_BCAST_RANKS: automatic
    1,   // DDL_TUNE_REDUCE_NT_LOAD: on
    24,  // DDL_TUNE_FUSED_NT_LOAD_MAX_P
    0,   // DDL_TUNE_ANCHOR: automatic
    1,   // DDL_TUNE_FUSED_BATCH
    4,   // DDL_TUNE_REDUCE_BATCH
    1,   // DDL_TUNE_BCAST_TILES
    0,   // DDL_TUNE_BCAST_XCD: off
    2,   // DDL_TUNE_UPDATE_REPS
    4,   // DDL_TUNE_UPDATE_BATCH
    16,  // DDL_TUNE_REDUCE_RANKS_MIN_P
    2,   // DDL_TUNE_BCAST_STORE_WAIT: binary32
    2,   // DDL_TUNE_FUSED_STORE_WAIT: large binary32 groups, 8 ranks on
};
static_assert(sizeof(kTuneDefault) / sizeof(kTuneDefault[0]) == DDL_TUNE_COUNT,
              "one default per knob");
std::atomic<int> g_tune[DDL_TUNE_COUNT];

namespace ddl {
int tuning(int knob) {
    if (knob < 0 || knob >= DDL_TUNE_COUNT)
        return 0;
    const int v = g_tune[knob].load(std::memory_order_relaxed);
    return v == 0 ? kTuneDefault[knob] : v - 1;
}
}  // namespace ddl
constexpr int kLaunchKinds = DDL_K_COUNT;

// One element type's share of a plan: its schedule and the device copies of
// the tables of the plan's mode.
struct Part {
    Schedule s;
    DevItem *d_items = nullptr;
    uint32_t *d_prefix = nullptr;
    std::vector<size_t> item_base, prefix_base;  // per step, into the above
    DevSpan *d_spans = nullptr;
    uint32_t *d_span_prefix = nullptr;
    uint32_t *d_span_of_tile = nullptr;
    uint8_t *d_chains = nullptr;
    uint32_t *d_tiny = nullptr;
    DevSpan *d_bk_spans = nullptr;
    uint32_t *d_bk_prefix = nullptr;
    uint32_t *d_bk_of_tile = nullptr;
    uint32_t *d_bk_span_tiles = nullptr;  // [b] first fused tile of bucket b, nb+1
    double *d_lars_partial = nullptr;  // LARS: two sums per tile (bucket-table
                                       // tiles, or fused tiles in the two-kernel form)
    float *d_lars_rate = nullptr;      // LARS: one rate per bucket
    void *d_sgd_home = nullptr;        // SGD without kept gradients, two-kernel
                                       // form: the reduced values (n elements)
};

struct ddl_plan_s {
    // one part per element type (a plain plan has one); buckets are issued
    // in list order, entry i naming (part, bucket within that part)
    std::vector<Part> parts;
    std::vector<std::pair<int, int>> order;
    bool typed = false;     // created with typed buckets (byte offsets)
    int mode = DDL_FUSED;
    size_t coalesce_bytes = 0;
    // the caller records the ready events in list order on one stream: a
    // group then waits for its last event only
    bool ordered_events = false;
    int nside = 0;          // side streams event-gated groups alternate over (0 auto)
    int fused_passes = 0;   // 0 automatic, 1 one kernel, 2 reduce + broadcast
    int step_form = 0;      // 0 automatic, 1 a launch per step, 2 persistent

    std::mutex mu;
    int device = -1;        // bound at first execution
    hipStream_t side[kMaxSideStreams] = {};
    hipEvent_t side_done[kMaxSideStreams] = {};
    hipEvent_t call_ev = nullptr;
    // the end of the latest call on each stream a call ended on: calls on
    // one stream complete in order, calls on different streams need one
    // event each, or a plan could be freed under an earlier call's kernels
    std::vector<std::pair<hipStream_t, hipEvent_t>> last_ev;
    // typed plans: a group's smaller element-type passes run on part_side,
    // forked from and joined back into the group's stream
    hipStream_t part_side = nullptr;
    hipEvent_t part_fork = nullptr, part_join = nullptr;
    // events made at binding for last_ev entries of streams first seen later
    // (the allocation-free entry point creates none)
    std::vector<hipEvent_t> spare_ev;
    bool in_flight = false;
    // an execution was enqueued on a stream under HIP graph capture: the
    // graph holds the addresses of this plan's tables, and its replays are
    // invisible to the event queries of busy(), so the one-shot cache never
    // destroys such a plan
    bool captured = false;
    // freed by ddl_plan_destroy: a call that looked the handle up before the
    // destroy finds this under the plan's mutex and enqueues nothing
    bool dead = false;

    // profiling: every launch of every prof_stride-th group is bracketed
    bool profiling = false;
    int prof_stride = 1;
    uint64_t prof_group = 0;        // groups seen since profiling was set
    std::vector<hipEvent_t> prof;   // pairs (start, end)
    std::vector<int> prof_kind;     // ddl_launch_kind of each pair
    int prof_used = 0;
};

namespace {

// ---------------------------------------------------------------------------
// device state
// ---------------------------------------------------------------------------
template <class T>
int upload(T **dst, const T *src, size_t count) {
    if (count == 0) {
        *dst = nullptr;
        return DDL_OK;
    }
    if (hipMalloc((void **)dst, count * sizeof(T)) != hipSuccess)
        return DDL_E_NOMEM;
    if (hipMemcpy(*dst, src, count * sizeof(T), hipMemcpyHostToDevice) != hipSuccess)
        return DDL_E_HIP;
    return DDL_OK;
}

void release_device(ddl_plan p) {
    if (p->device < 0)
        return;
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(p->device);
    for (Part &pt : p->parts) {
        (void)hipFree(pt.d_items);
        (void)hipFree(pt.d_prefix);
        (void)hipFree(pt.d_spans);
        (void)hipFree(pt.d_span_prefix);
        (void)hipFree(pt.d_span_of_tile);
        (void)hipFree(pt.d_chains);
        (void)hipFree(pt.d_tiny);
        (void)hipFree(pt.d_bk_spans);
        (void)hipFree(pt.d_bk_prefix);
        (void)hipFree(pt.d_bk_of_tile);
        (void)hipFree(pt.d_bk_span_tiles);
        (void)hipFree(pt.d_lars_partial);
        (void)hipFree(pt.d_lars_rate);
        (void)hipFree(pt.d_sgd_home);
        pt = Part{std::move(pt.s)};
    }
    for (hipEvent_t e : p->prof)
        (void)hipEventDestroy(e);
    if (p->call_ev)
        (void)hipEventDestroy(p->call_ev);
    for (auto &se : p->last_ev)
        (void)hipEventDestroy(se.second);
    p->last_ev.clear();
    for (hipEvent_t e : p->spare_ev)
        (void)hipEventDestroy(e);
    p->spare_ev.clear();
    if (p->part_fork)
        (void)hipEventDestroy(p->part_fork);
    if (p->part_join)
        (void)hipEventDestroy(p->part_join);
    if (p->part_side)
        (void)hipStreamDestroy(p->part_side);
    p->call_ev = p->part_fork = p->part_join = nullptr;
    p->part_side = nullptr;
    for (int i = 0; i < kMaxSideStreams; ++i) {
        if (p->side_done[i])
            (void)hipEventDestroy(p->side_done[i]);
        if (p->side[i])
            (void)hipStreamDestroy(p->side[i]);
        p->side[i] = nullptr;
        p->side_done[i] = nullptr;
    }
    (void)hipSetDevice(cur);
    p->device = -1;
}

int bind_device(ddl_plan p, int dev) {
    p->device = dev;
    // default-priority streams only
    for (int i = 0; i < kMaxSideStreams; ++i)
        if (hipStreamCreateWithFlags(&p->side[i], hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&p->side_done[i], hipEventDisableTiming) != hipSuccess)
            return DDL_E_HIP;
    if (hipEventCreateWithFlags(&p->call_ev, hipEventDisableTiming) != hipSuccess)
        return DDL_E_HIP;
    for (int i = 0; i < kSpareEvents; ++i) {
        hipEvent_t e;
        if (hipEventCreateWithFlags(&e, kTrackEventFlags) != hipSuccess)
            return DDL_E_HIP;
        p->spare_ev.push_back(e);
    }
    if (p->parts.size() > 1 &&
        (hipStreamCreateWithFlags(&p->part_side, hipStreamNonBlocking) != hipSuccess ||
         hipEventCreateWithFlags(&p->part_fork, hipEventDisableTiming) != hipSuccess ||
         hipEventCreateWithFlags(&p->part_join, hipEventDisableTiming) != hipSuccess))
        return DDL_E_HIP;
    for (Part &pt : p->parts) {
        const Schedule &s = pt.s;
        int rc = DDL_OK;
        if (p->mode == DDL_STEPWISE) {
            std::vector<DevItem> items;
            std::vector<uint32_t> prefix;
            for (int st = 0; st < s.nsteps; ++st) {
                pt.item_base.push_back(items.size());
                pt.prefix_base.push_back(prefix.size());
                items.insert(items.end(), s.items[st].begin(), s.items[st].end());
                prefix.insert(prefix.end(), s.prefix[st].begin(), s.prefix[st].end());
            }
            if ((rc = upload(&pt.d_items, items.data(), items.size())) ||
                (rc = upload(&pt.d_prefix, prefix.data(), prefix.size())))
                return rc;
        }
        // the fused tables are small; stepwise plans keep them for the
        // one-rank SGD step, which has no schedule step to ride on, and the
        // bucket tables for the broadcast and the LARS step
        if ((rc = upload(&pt.d_spans, s.spans.data(), s.spans.size())) ||
            (rc = upload(&pt.d_span_prefix, s.span_prefix.data(), s.span_prefix.size())) ||
            (rc = upload(&pt.d_span_of_tile, s.span_of_tile.data(), s.span_of_tile.size())) ||
            (rc = upload(&pt.d_chains, s.chains.data(), s.chains.size())) ||
            (rc = upload(&pt.d_tiny, s.tiny.data(), s.tiny.size())) ||
            (rc = upload(&pt.d_bk_spans, s.bk_spans.data(), s.bk_spans.size())) ||
            (rc = upload(&pt.d_bk_prefix, s.bk_prefix.data(), s.bk_prefix.size())) ||
            (rc = upload(&pt.d_bk_of_tile, s.bk_of_tile.data(), s.bk_of_tile.size())))
            return rc;
        std::vector<uint32_t> bst(s.buckets.size() + 1, 0);
        for (size_t b = 0; b <= s.buckets.size(); ++b)
            bst[b] = s.span_prefix[s.span_at[b]];
        if ((rc = upload(&pt.d_bk_span_tiles, bst.data(), bst.size())))
            return rc;
    }
    return DDL_OK;
}

// ---------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------
// A grid holds at most 2^32 - 1 work-items in x: cut bigger launches.
constexpr uint32_t kMaxTilesPerLaunch = 1u << 23;

// Form of the fused pass of a group of `elems` elements per rank: one
// kernel, or a reduce kernel that writes rank 0 and a broadcast kernel (see
// fused_kernel.hip).  Automatic: two kernels from 16 ranks on, for groups
// of at least 200 MB over all ranks (binary32; 400 MB binary16).  Measured
// on MI355X: whole workloads (paired, six repeats) 40 ranks fp32 +5..+18%,
// 16 ranks fp32 ResNet-50 multi-ring +7.3%, 16 ranks fp16 torus (818 MB)
// +5.8%; 8 ranks -3%.  By group size, one bucket per call: 40 ranks fp32
// two kernels win from 8 MB per rank (-7%), lose at 4 MB (+4%) and below;
// 16 ranks fp32 win from 16 MB (-3%), lose at 8 MB (+4%) and below (+16..19%,
// launch-bound); 16 ranks fp16 still lose at 16 MB (+8%).  With the SGD
// step, the one-kernel form updates the weights in its epilogue; the
// two-kernel form reduces to rank 0 and its broadcast steps the replicas as
// it copies, or, when the gradients are not kept, reduces to a scratch
// buffer and runs the update kernel from it.
constexpr uint64_t kTwoKernelMinBytes = 200ull << 20;
int fused_passes(ddl_plan p, const Schedule &s, uint64_t elems) {
    if (s.P < 2)
        return 1;
    if (p->fused_passes)
        return p->fused_passes;
    const uint64_t min_bytes = kTwoKernelMinBytes * (s.esz == 4 ? 1 : 2);
    return s.P >= 16 && (uint64_t)s.P * elems * (uint64_t)s.esz >= min_bytes ? 2 : 1;
}

// Form of a stepwise group: one launch per schedule step (1), or one
// persistent launch whose workgroups each walk every step of one tile (2).
// Automatic: persistent, which measured faster on every workload on MI355X
// (ms per all-reduce, per-step launches against persistent: 40 ranks x 300M
// in 64 event-gated buckets 43.5 / 25.5; 8 ranks x 300M 6.93 / 3.97;
// ResNet-50 over 16 ranks and 4 rings 1.47 / 0.74; the binary16 4x4 torus
// 0.66 / 0.43; 4 ranks x 2^20 0.024 / 0.011): a tile's intermediate values
// are re-read while they are still in the caches, and a group costs one
// dispatch instead of 2 (P - 1).  The SGD step rides on either form.
int step_form(ddl_plan p, const Schedule &, uint64_t) {
    return p->step_form ? p->step_form : 2;
}

// Side streams event-gated groups alternate over.  Automatic: two for
// stepwise plans and for fused plans with small buckets, where the next
// group's launches fill the previous group's ramp-down (measured on MI355X
// with one event per bucket: 40 ranks stepwise 43.7 ms against 55.7; the
// ResNet-50 multi-ring fused 1.49 ms against 2.65, stepwise 12.1 against
// 18.6); one for fused plans with large buckets, whose launches each fill
// the chip (40 ranks x 18.75 MB buckets: 16.9 ms against 17.2 with two).
int side_streams(ddl_plan p) {
    if (p->nside)
        return p->nside;
    if (p->mode == DDL_STEPWISE)
        return 2;
    uint64_t bytes = 0, count = 0;
    for (const Part &pt : p->parts) {
        for (const Bucket &b : pt.s.buckets)
            bytes += b.len * (uint64_t)pt.s.esz;
        count += pt.s.buckets.size();
    }
    const uint64_t mean_bytes = count ? bytes / count : 0;
    return mean_bytes < (4ull << 20) ? 2 : 1;
}

// Ranks one broadcast workgroup writes (knob DDL_TUNE_BCAST_RANKS, 0 =
// automatic).  Measured on MI355X (paired runs): 40 ranks fp32, two (5.45
// TB/s; 4 within 1%, all 39 -4%, one -7%); 16 ranks, seven (fp32 5.66
// against 5.58 with three and 5.47 with all 15; fp16 5.48 against 5.40 and
// 5.38).
int bcast_ranks_per_group(int P) {
    const int v = tuning(DDL_TUNE_BCAST_RANKS);
    if (v > 0)
        return std::min(v, std::max(P - 1, 1));
    if (P >= 32)
        return 2;
    return std::min(7, std::max(P - 1, 1));
}

// The LARS step's arguments of one call (ddl_plan_execute_lars).
struct LarsCall {
    RankPtrs w;
    int nweights;
    float lr;
    double coeff, eps;
    float *rates_out;
    // the partial sums and rates, when not the plan's own buffers
    double *partial;
    float *rate;
};

struct Launcher {
    ddl_plan p;
    const RankPtrs &bufs;
    hipStream_t stream;
    const SgdArgs *sgd;  // null for the plain all-reduce
    const LarsCall *lars = nullptr;  // the LARS step after the all-reduce
    Part *pt = nullptr;  // the element type of the current group
    std::vector<Bucket> runs;
    bool prof = false;   // bracket the launches of the current group
    bool lars_done = false;  // the group's LARS step rode on its fused pass

    int bracket_begin(int kind) {
        if (!prof)
            return DDL_OK;
        if ((size_t)(2 * p->prof_used + 2) > p->prof.size()) {
            hipEvent_t a, b;
            if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess)
                return DDL_E_HIP;
            p->prof.push_back(a);
            p->prof.push_back(b);
            p->prof_kind.push_back(0);
        }
        p->prof_kind[p->prof_used] = kind;
        return hipEventRecord(p->prof[2 * p->prof_used], stream) == hipSuccess ? DDL_OK
                                                                               : DDL_E_HIP;
    }
    int bracket_end() {
        if (!prof)
            return DDL_OK;
        if (hipEventRecord(p->prof[2 * p->prof_used + 1], stream) != hipSuccess)
            return DDL_E_HIP;
        ++p->prof_used;
        return DDL_OK;
    }

    int step(int st, uint32_t lo, uint32_t hi) {
        const Schedule &s = pt->s;
        if (lo == hi)
            return DDL_OK;
        const uint32_t *pre = s.prefix[st].data();
        StepArgs a;
        a.items = pt->d_items + pt->item_base[st];
        a.prefix = pt->d_prefix + pt->prefix_base[st];
        a.item_lo = lo;
        a.item_hi = hi;
        a.divisor = (float)s.P;
        a.anchor = s.step_anchor;
        for (uint32_t t = pre[lo]; t < pre[hi]; t += kMaxTilesPerLaunch) {
            const uint32_t tiles = std::min(kMaxTilesPerLaunch, pre[hi] - t);
            a.tile_base = t;
            int rc = bracket_begin(s.step_kind[st]);
            if (rc)
                return rc;
            if (launch_step(s.dtype, s.step_kind[st], s.step_vpl, bufs, a, sgd, tiles, stream) !=
                hipSuccess)
                return DDL_E_HIP;
            if ((rc = bracket_end()))
                return rc;
        }
        return DDL_OK;
    }

    // the persistent step kernel over the fused tiles of buckets [b0, b1)
    int walk(int b0, int b1) {
        const Schedule &s = pt->s;
        const uint32_t lo = s.span_at[b0], hi = s.span_at[b1];
        if (lo == hi)
            return DDL_OK;
        const uint32_t *pre = s.span_prefix.data();
        FusedArgs a;
        std::memset(&a, 0, sizeof(a));
        a.spans = pt->d_spans;
        a.prefix = pt->d_span_prefix;
        a.tile_span = pt->d_span_of_tile;
        a.chains = pt->d_chains;
        a.span_lo = lo;
        a.span_hi = hi;
        a.P = s.P;
        a.group = s.group;
        a.mean = s.op == DDL_MEAN;
        a.divisor = (float)s.P;
        a.anchor = s.fused_anchor;
        for (uint32_t t = pre[lo]; t < pre[hi]; t += kMaxTilesPerLaunch) {
            const uint32_t tiles = std::min(kMaxTilesPerLaunch, pre[hi] - t);
            a.tile_base = t;
            a.tile_end = t + tiles;
            int rc = bracket_begin(DDL_K_WALK);
            if (rc)
                return rc;
            if (launch_walk(s.dtype, bufs, a, sgd, tiles, stream) != hipSuccess)
                return DDL_E_HIP;
            if ((rc = bracket_end()))
                return rc;
        }
        return DDL_OK;
    }

    // the fused pass of buckets [b0, b1): one kernel, or the reduce kernel
    // over their spans and then the broadcast over the runs of memory they
    // cover (and, with the SGD step, the update kernel)
    int fused(int b0, int b1) {
        const Schedule &s = pt->s;
        const uint32_t lo = s.span_at[b0], hi = s.span_at[b1];
        if (lo == hi)
            return DDL_OK;
        const uint32_t *pre = s.span_prefix.data();
        FusedArgs a;
        a.spans = pt->d_spans;
        a.prefix = pt->d_span_prefix;
        a.tile_span = pt->d_span_of_tile;
        a.chains = pt->d_chains;
        a.span_lo = lo;
        a.span_hi = hi;
        a.P = s.P;
        a.group = s.group;
        a.mean = s.op == DDL_MEAN;
        a.divisor = (float)s.P;
        a.anchor = s.fused_anchor;
        uint64_t elems = 0;
        for (int b = b0; b < b1; ++b)
            elems += s.buckets[b].len;
        const bool two = fused_passes(p, s, elems) == 2;
        if (!two && !sgd && s.tiny_prefix[hi] - s.tiny_prefix[lo] == hi - lo) {
            // every span of the group is tiny: one wave per span
            TinyArgs ta;
            ta.spans = pt->d_spans;
            ta.tiny = pt->d_tiny;
            ta.chains = pt->d_chains;
            ta.lo = s.tiny_prefix[lo];
            ta.hi = s.tiny_prefix[hi];
            ta.P = s.P;
            ta.group = s.group;
            ta.mean = s.op == DDL_MEAN;
            ta.divisor = (float)s.P;
            int rc = bracket_begin(DDL_K_FUSED);
            if (rc)
                return rc;
            if (launch_tiny(s.dtype, bufs, ta, stream) != hipSuccess)
                return DDL_E_HIP;
            return bracket_end();
        }
        // two-kernel SGD without kept gradients: the results go to the
        // plan's scratch buffer, and the gradient buffers stay as they were
        const bool scratch = two && sgd && !sgd->keep_grads;
        a.home = scratch ? pt->d_sgd_home : bufs.p[0];
        // the LARS step in the two-kernel form: the reduce kernel also sums
        // the squares of each tile, a rate kernel turns the sums into the
        // buckets' rates, and the broadcast steps the replicas
        const bool fused_lars = two && lars;
        a.partial = nullptr;
        a.w0 = nullptr;
        if (fused_lars) {
            a.partial = lars->partial ? lars->partial : pt->d_lars_partial;
            a.w0 = static_cast<const float *>(lars->w.p[0]);
        }
        for (uint32_t t = pre[lo]; t < pre[hi]; t += kMaxTilesPerLaunch) {
            const uint32_t tiles = std::min(kMaxTilesPerLaunch, pre[hi] - t);
            a.tile_base = t;
            a.tile_end = t + tiles;
            int rc = bracket_begin(two ? DDL_K_FUSED_REDUCE : DDL_K_FUSED);
            if (rc)
                return rc;
            if (launch_fused(s.dtype, bufs, a, two ? nullptr : sgd, two, tiles, stream) !=
                hipSuccess)
                return DDL_E_HIP;
            if ((rc = bracket_end()))
                return rc;
        }
        if (!two)
            return DDL_OK;
        if (fused_lars)
            return lars_pass_tail(b0, b1, a.partial);
        if (scratch)
            return update(b0, b1, a.home, nullptr, sgd->lr, sgd->w, sgd->nweights);
        // with the SGD step, the broadcast steps the replicas as it copies
        return sgd ? bcast_update(b0, b1, nullptr, sgd->lr, sgd->w, sgd->nweights)
                   : broadcast(b0, b1);
    }

    // the broadcast of buckets [b0, b1) over the bucket table, whose
    // workgroups also step the weight replicas w with each bucket's rate
    // (rate null: the constant lr)
    int bcast_update(int b0, int b1, const float *rate, float lr, const RankPtrs &w,
                     int nweights) {
        const Schedule &s = pt->s;
        BcastArgs bc;
        std::memset(&bc, 0, sizeof(bc));
        bc.P = s.P;
        bc.ranks_per_group = bcast_ranks_per_group(s.P);
        bc.ngroups = (s.P - 1 + bc.ranks_per_group - 1) / bc.ranks_per_group;
        bc.tiles_per_group = 1;
        bc.nxcd = 1;
        bc.spans = pt->d_bk_spans;
        bc.prefix = pt->d_bk_prefix;
        bc.tile_span = pt->d_bk_of_tile;
        bc.rate = rate;
        bc.lr = lr;
        bc.nweights = nweights;
        const uint32_t *bp = s.bk_prefix.data();
        const uint32_t max_tiles = 0xffffffu / (uint32_t)bc.ngroups;
        for (uint32_t t = bp[b0]; t < bp[b1]; t += max_tiles) {
            bc.tile_base = t;
            bc.tile_end = std::min(bp[b1], t + max_tiles);
            int rc = bracket_begin(DDL_K_BROADCAST);
            if (rc)
                return rc;
            if (launch_bcast_update(s.dtype, bufs, w, bc, stream) != hipSuccess)
                return DDL_E_HIP;
            if ((rc = bracket_end()))
                return rc;
        }
        return DDL_OK;
    }

    // after the LARS reduce kernel of buckets [b0, b1): the rates from the
    // fused tiles' partial sums, then the broadcast that steps the replicas
    int lars_pass_tail(int b0, int b1, double *partial) {
        const Schedule &s = pt->s;
        LarsArgs la = update_args(b0, b1, bufs.p[0], lars->rate ? lars->rate : pt->d_lars_rate,
                                  lars->lr, lars->nweights);
        la.prefix = pt->d_bk_span_tiles;   // the buckets' fused-tile ranges
        la.partial = partial;
        la.rate_out = lars->rates_out;
        la.coeff = lars->coeff;
        la.eps = lars->eps;
        int rc = bracket_begin(DDL_K_LARS_RATE);
        if (rc)
            return rc;
        if (launch_lars(s.dtype, DDL_K_LARS_RATE, lars->w, la, (uint32_t)(b1 - b0), stream) !=
            hipSuccess)
            return DDL_E_HIP;
        if ((rc = bracket_end()))
            return rc;
        if ((rc = bcast_update(b0, b1, la.rate, 0.0f, lars->w, lars->nweights)))
            return rc;
        lars_done = true;
        return DDL_OK;
    }

    // the broadcast of buckets [b0, b1) from rank 0 to ranks 1..P-1
    int broadcast(int b0, int b1) {
        const Schedule &s = pt->s;
        runs.clear();
        for (int b = b0; b < b1; ++b)
            if (s.buckets[b].len)
                runs.push_back(s.buckets[b]);
        std::sort(runs.begin(), runs.end(),
                  [](const Bucket &x, const Bucket &y) { return x.off < y.off; });
        size_t m = 0;
        for (size_t i = 1; i < runs.size(); ++i) {
            if (runs[m].off + runs[m].len == runs[i].off)
                runs[m].len += runs[i].len;
            else
                runs[++m] = runs[i];
        }
        runs.resize(runs.empty() ? 0 : m + 1);
        BcastArgs bc;
        std::memset(&bc, 0, sizeof(bc));
        bc.P = s.P;
        bc.ranks_per_group = bcast_ranks_per_group(s.P);
        bc.ngroups = (s.P - 1 + bc.ranks_per_group - 1) / bc.ranks_per_group;
        bc.tiles_per_group = std::max(1, std::min(tuning(DDL_TUNE_BCAST_TILES), 64));
        bc.nxcd = std::max(1, std::min(tuning(DDL_TUNE_BCAST_XCD), 64));
        // a grid holds at most 2^32 - 1 work-items: runs are cut at
        // multiples of max_elems, which keeps the tiles' anchoring (the
        // broadcast always anchors: its runs are whole buckets)
        const uint64_t tile = fused_tile_elems(s.esz);
        // (the die-dealt order pads the last nxcd-block: keep headroom)
        const uint32_t max_tiles = 0xffffffu / (uint32_t)(bc.ngroups * bc.nxcd) *
                                   (uint32_t)bc.nxcd;
        const uint64_t max_elems = (uint64_t)max_tiles * tile;
        if (runs.size() > 1) {
            // not one run of memory: one launch over the buckets' table
            bc.spans = pt->d_bk_spans;
            bc.prefix = pt->d_bk_prefix;
            bc.tile_span = pt->d_bk_of_tile;
            const uint32_t *bp = s.bk_prefix.data();
            for (uint32_t t = bp[b0]; t < bp[b1]; t += max_tiles) {
                bc.tile_base = t;
                bc.tile_end = std::min(bp[b1], t + max_tiles);
                int rc = bracket_begin(DDL_K_BROADCAST);
                if (rc)
                    return rc;
                if (launch_bcast(s.dtype, bufs, bc, stream) != hipSuccess)
                    return DDL_E_HIP;
                if ((rc = bracket_end()))
                    return rc;
            }
            return DDL_OK;
        }
        for (const Bucket &r : runs) {
            for (uint64_t o = r.off; o < r.off + r.len; o = (o / max_elems + 1) * max_elems) {
                bc.off = o;
                bc.len = std::min((o / max_elems + 1) * max_elems, r.off + r.len) - o;
                bc.aligned = bc.off % s.q == 0;
                int rc = bracket_begin(DDL_K_BROADCAST);
                if (rc)
                    return rc;
                if (launch_bcast(s.dtype, bufs, bc, stream) != hipSuccess)
                    return DDL_E_HIP;
                if ((rc = bracket_end()))
                    return rc;
            }
        }
        return DDL_OK;
    }

    // Arguments of the update and LARS kernels over buckets [b0, b1): y the
    // reduced values, rate null for the constant rate lr
    LarsArgs update_args(int b0, int b1, const void *y, float *rate, float lr, int nweights) {
        LarsArgs a;
        std::memset(&a, 0, sizeof(a));
        a.spans = pt->d_bk_spans;
        a.prefix = pt->d_bk_prefix;
        a.tile_span = pt->d_bk_of_tile;
        a.y = y;
        a.rate = rate;
        a.lr = lr;
        a.nweights = nweights;
        // replicas per update workgroup: measured on MI355X, 40 replicas x
        // 18.75 MB buckets, paired: 2 per workgroup 279 us per launch, 1
        // 287, 4 297, 8 291, all 40 302 (load batch 1-8 within 1% at 2)
        const int g = tuning(DDL_TUNE_UPDATE_REPS);
        a.reps_per_group = g > 0 ? std::min(g, nweights) : nweights;
        a.ngroups = (nweights + a.reps_per_group - 1) / a.reps_per_group;
        a.bucket_lo = (uint32_t)b0;
        a.bucket_hi = (uint32_t)b1;
        return a;
    }

    // one launch kind over the bucket-table tiles of buckets [b0, b1)
    int table_tiles(int kind, int b0, int b1, LarsArgs &a, const RankPtrs &w) {
        const uint32_t *bp = pt->s.bk_prefix.data();
        for (uint32_t t = bp[b0]; t < bp[b1]; t += kMaxTilesPerLaunch) {
            a.tile_base = t;
            a.tile_end = std::min(bp[b1], t + kMaxTilesPerLaunch);
            int rc = bracket_begin(kind);
            if (rc)
                return rc;
            if (launch_lars(pt->s.dtype, kind, w, a, a.tile_end - t, stream) != hipSuccess)
                return DDL_E_HIP;
            if ((rc = bracket_end()))
                return rc;
        }
        return DDL_OK;
    }

    // w = w - rate * y on every replica over buckets [b0, b1)
    int update(int b0, int b1, const void *y, float *rate, float lr, const RankPtrs &w,
               int nweights) {
        LarsArgs a = update_args(b0, b1, y, rate, lr, nweights);
        return table_tiles(DDL_K_UPDATE, b0, b1, a, w);
    }

    // the LARS step of buckets [b0, b1), once their all-reduce is enqueued:
    // the norms of every tile, the rate of every bucket, the update
    int lars_step(int b0, int b1) {
        LarsArgs a = update_args(b0, b1, bufs.p[0], lars->rate ? lars->rate : pt->d_lars_rate,
                                 lars->lr, lars->nweights);
        a.partial = lars->partial ? lars->partial : pt->d_lars_partial;
        a.rate_out = lars->rates_out;
        a.coeff = lars->coeff;
        a.eps = lars->eps;
        int rc = table_tiles(DDL_K_LARS_NORM, b0, b1, a, lars->w);
        if (rc || b1 == b0)
            return rc;
        if ((rc = bracket_begin(DDL_K_LARS_RATE)))
            return rc;
        if (launch_lars(pt->s.dtype, DDL_K_LARS_RATE, lars->w, a, (uint32_t)(b1 - b0), stream) !=
            hipSuccess)
            return DDL_E_HIP;
        if ((rc = bracket_end()))
            return rc;
        return table_tiles(DDL_K_UPDATE, b0, b1, a, lars->w);
    }

    // every launch of buckets [b0, b1)
    int group(int b0, int b1) {
        const Schedule &s = pt->s;
        int rc = DDL_OK;
        lars_done = false;
        if (p->mode == DDL_FUSED || (sgd && s.P == 1)) {
            rc = fused(b0, b1);
        } else {
            uint64_t elems = 0;
            for (int b = b0; b < b1; ++b)
                elems += s.buckets[b].len;
            if (s.nsteps > 0 && step_form(p, s, elems) == 2)
                rc = walk(b0, b1);
            else
                for (int st = 0; st < s.nsteps && !rc; ++st)
                    rc = step(st, s.item_at[st][b0], s.item_at[st][b1]);
        }
        if (rc || !lars || lars_done)
            return rc;
        return lars_step(b0, b1);
    }
};

// The scratch buffer of two-kernel SGD without kept gradients (n elements
// per part), allocated by the first such call.
int ensure_sgd_home(ddl_plan p) {
    for (Part &pt : p->parts) {
        if (pt.d_sgd_home || pt.s.n == 0)
            continue;
        if (hipMalloc(&pt.d_sgd_home, (size_t)pt.s.n * (size_t)pt.s.esz) != hipSuccess)
            return DDL_E_NOMEM;
    }
    return DDL_OK;
}

// Tiles whose partial sums the LARS step keeps: the bucket table's (the norm
// kernel's) or the fused tables' (the two-kernel form's reduce kernel).
size_t lars_tiles(const Schedule &s) {
    const size_t bk = s.bk_prefix.empty() ? 0 : s.bk_prefix.back();
    const size_t sp = s.span_prefix.empty() ? 0 : s.span_prefix.back();
    return std::max(bk, sp);
}

// Device memory of the LARS step, allocated by a plan's first LARS call.
int ensure_lars(ddl_plan p) {
    for (Part &pt : p->parts) {
        if (pt.d_lars_partial)
            continue;
        const size_t tiles = std::max<size_t>(1, lars_tiles(pt.s));
        const size_t nb = std::max<size_t>(1, pt.s.buckets.size());
        if (hipMalloc((void **)&pt.d_lars_partial, 2 * tiles * sizeof(double)) != hipSuccess)
            return DDL_E_NOMEM;
        if (hipMalloc((void **)&pt.d_lars_rate, nb * sizeof(float)) != hipSuccess)
            return DDL_E_NOMEM;
    }
    return DDL_OK;
}

// The event that records the end of the latest call on stream ls: an
// existing entry, else one of the events made at binding, else (unless the
// caller may not allocate) a new one.  Null on failure.
hipEvent_t *last_event(ddl_plan p, hipStream_t ls, bool may_create = true) {
    for (auto &se : p->last_ev)
        if (se.first == ls)
            return &se.second;
    hipEvent_t e = nullptr;
    if (!p->spare_ev.empty()) {
        e = p->spare_ev.back();
        p->spare_ev.pop_back();
    } else if (!may_create || hipEventCreateWithFlags(&e, kTrackEventFlags) != hipSuccess) {
        return nullptr;
    }
    p->last_ev.emplace_back(ls, e);
    return &p->last_ev.back().second;
}

// The end (one past the last bucket, in list order) of the group that
// starts at bucket b0: consecutive buckets with equal ready events, then,
// with a threshold, following buckets until the group holds coalesce_bytes
// per rank.  ready == nullptr: every event is NULL (equal); distinct: every
// bucket's event differs from the others' (the grouping a caller gets with
// one event per bucket).
int group_end(const ddl_plan_s *p, void *const *ready, int b0, bool distinct = false) {
    const int nb = (int)p->order.size();
    auto bucket_bytes = [&](int i) {
        const Part &pt = p->parts[p->order[i].first];
        return (size_t)pt.s.buckets[p->order[i].second].len * (size_t)pt.s.esz;
    };
    void *ev0 = ready ? ready[b0] : nullptr;
    int b1 = b0 + 1;
    size_t bytes = bucket_bytes(b0);
    while (b1 < nb) {
        const bool same = !distinct && (ready ? ready[b1] : nullptr) == ev0;
        if (!same && !(p->coalesce_bytes && bytes < p->coalesce_bytes))
            break;
        bytes += bucket_bytes(b1);
        ++b1;
    }
    return b1;
}

// noalloc: the allocation-free entry point -- the plan must be bound, the
// LARS buffers come in through lars, no event is created and no launch is
// bracketed for profiling.
int execute_locked(ddl_plan p, void *const *bufs, void *const *ready, void *stream_,
                   void *done_event, const SgdArgs *sgd, const LarsCall *lars = nullptr,
                   bool noalloc = false) {
    const int P = p->parts[0].s.P;
    bool any_elems = false;
    for (const Part &pt : p->parts)
        any_elems = any_elems || pt.s.n > 0;
    for (int r = 0; r < P; ++r) {
        if (!bufs[r] && any_elems)
            return DDL_E_NULL;
        if ((uintptr_t)bufs[r] % kVecBytes)
            return DDL_E_ALIGN;
    }
    for (int r = 0; sgd && r < sgd->nweights; ++r) {
        if (!sgd->w.p[r] && any_elems)
            return DDL_E_NULL;
        if ((uintptr_t)sgd->w.p[r] % kVecBytes)
            return DDL_E_ALIGN;
    }
    for (int r = 0; lars && r < lars->nweights; ++r) {
        if (!lars->w.p[r] && any_elems)
            return DDL_E_NULL;
        if ((uintptr_t)lars->w.p[r] % kVecBytes)
            return DDL_E_ALIGN;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return DDL_E_HIP;
    if (p->device < 0) {
        if (noalloc)
            return DDL_E_UNBOUND;
        int rc = bind_device(p, dev);
        if (rc) {
            release_device(p);
            return rc;
        }
    } else if (p->device != dev) {
        return DDL_E_DEVICE;
    }
    if (lars && !lars->partial) {
        int rc = ensure_lars(p);
        if (rc)
            return rc;
    }
    if (sgd && !sgd->keep_grads && p->mode == DDL_FUSED &&
        fused_passes(p, p->parts[0].s, p->parts[0].s.n) == 2) {
        int rc = ensure_sgd_home(p);
        if (rc)
            return rc;
    }
    RankPtrs rp;
    std::memset(&rp, 0, sizeof(rp));
    for (int r = 0; r < P; ++r)
        rp.p[r] = bufs[r];

    hipStream_t cs = static_cast<hipStream_t>(stream_);
    // under HIP graph capture the graph keeps this plan's table addresses
    // for its replays (a stream the runtime cannot query counts as not
    // capturing; its error is cleared so that no launch reports it)
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(cs, &cap) != hipSuccess) {
        (void)hipGetLastError();
        cap = hipStreamCaptureStatusNone;
    }
    if (cap == hipStreamCaptureStatusActive)
        p->captured = true;
    const int nb = (int)p->order.size();
    bool any_event = false;
    for (int b = 0; ready && b < nb; ++b)
        any_event = any_event || ready[b] != nullptr;
    hipStream_t ls = any_event ? p->side[0] : cs;
    // the event that will mark the end of this call on ls (busy
    // tracking), taken before anything is enqueued: a call that cannot
    // track its work leaves none in flight
    hipEvent_t *last = last_event(p, ls, !noalloc);
    if (!last)
        return noalloc ? DDL_E_NOMEM : DDL_E_HIP;
    if (any_event && hipEventRecord(p->call_ev, cs) != hipSuccess)
        return DDL_E_HIP;

    Launcher L{p, rp, ls, sgd, lars};
    int b0 = 0, g = 0, used = 0;
    std::vector<std::pair<int, int>> range(p->parts.size());
    while (b0 < nb) {
        L.prof = !noalloc && p->profiling && p->prof_group++ % (uint64_t)p->prof_stride == 0;
        const int b1 = group_end(p, ready, b0);
        if (any_event) {
            // groups alternate over the side streams: independent buckets,
            // so one group's tail overlaps the next one's start
            const int si = g % side_streams(p);
            L.stream = p->side[si];
            used = std::max(used, si + 1);
            void *last = reinterpret_cast<void *>(1);
            // with ordered events the last event of the group implies the
            // earlier ones; buckets without an event still wait for the
            // caller's stream as of the call
            int from = b0;
            if (p->ordered_events) {
                int lastev = -1;
                bool anynull = false;
                for (int b = b0; b < b1; ++b) {
                    if (ready[b])
                        lastev = b;
                    else
                        anynull = true;
                }
                if (anynull && hipStreamWaitEvent(L.stream, p->call_ev, 0) != hipSuccess)
                    return DDL_E_HIP;
                from = lastev < 0 ? b1 : lastev;
            }
            for (int b = from; b < b1; ++b) {
                void *ev = ready[b] ? ready[b] : static_cast<void *>(p->call_ev);
                if (ev == last || (p->ordered_events && !ready[b]))
                    continue;
                if (hipStreamWaitEvent(L.stream, static_cast<hipEvent_t>(ev), 0) != hipSuccess)
                    return DDL_E_HIP;
                last = ev;
            }
        }
        // one pass (or one step sequence) per element type in the group:
        // the buckets of one type are numbered in list order, so those in
        // the group are a contiguous range of its part
        for (auto &r : range)
            r = {-1, -1};
        for (int b = b0; b < b1; ++b) {
            auto &r = range[p->order[b].first];
            if (r.first < 0)
                r.first = p->order[b].second;
            r.second = p->order[b].second + 1;
        }
        // with more than one element type in the group, the largest part
        // runs on the group's stream and the others on the plan's part
        // stream at the same time (the small binary32 tensors of a mixed
        // gradient are latency-bound: alone they leave the device idle)
        int big = -1, nparts = 0;
        size_t big_bytes = 0;
        for (size_t q = 0; q < p->parts.size(); ++q) {
            if (range[q].first < 0)
                continue;
            const Part &pq = p->parts[q];
            size_t bytes_q = 0;
            for (int b = range[q].first; b < range[q].second; ++b)
                bytes_q += (size_t)pq.s.buckets[b].len * (size_t)pq.s.esz;
            if (big < 0 || bytes_q > big_bytes) {
                big = (int)q;
                big_bytes = bytes_q;
            }
            ++nparts;
        }
        const hipStream_t gs = L.stream;
        if (nparts > 1 && (hipEventRecord(p->part_fork, gs) != hipSuccess ||
                           hipStreamWaitEvent(p->part_side, p->part_fork, 0) != hipSuccess))
            return DDL_E_HIP;
        for (size_t q = 0; q < p->parts.size(); ++q) {
            if (range[q].first < 0 || (nparts > 1 && (int)q == big))
                continue;
            L.pt = &p->parts[q];
            L.stream = nparts > 1 ? p->part_side : gs;
            int rc = L.group(range[q].first, range[q].second);
            if (rc)
                return rc;
        }
        if (nparts > 1) {
            if (hipEventRecord(p->part_join, p->part_side) != hipSuccess)
                return DDL_E_HIP;
            L.pt = &p->parts[big];
            L.stream = gs;
            int rc = L.group(range[big].first, range[big].second);
            if (rc)
                return rc;
            if (hipStreamWaitEvent(gs, p->part_join, 0) != hipSuccess)
                return DDL_E_HIP;
        }
        b0 = b1;
        ++g;
    }
    if (any_event) {
        // side stream 0 joins the others, then the caller's stream joins it
        for (int i = 1; i < used; ++i)
            if (hipEventRecord(p->side_done[i], p->side[i]) != hipSuccess ||
                hipStreamWaitEvent(p->side[0], p->side_done[i], 0) != hipSuccess)
                return DDL_E_HIP;
        if (hipEventRecord(p->side_done[0], p->side[0]) != hipSuccess ||
            hipStreamWaitEvent(cs, p->side_done[0], 0) != hipSuccess)
            return DDL_E_HIP;
    }
    if (done_event && hipEventRecord(static_cast<hipEvent_t>(done_event), ls) != hipSuccess)
        return DDL_E_HIP;
    if (hipEventRecord(*last, ls) != hipSuccess)
        return DDL_E_HIP;
    p->in_flight = true;
    return DDL_OK;
}

bool busy(ddl_plan p) {
    if (!p->in_flight || p->device < 0)
        return false;
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(p->device);
    bool pending = false;
    for (auto &se : p->last_ev)
        pending = pending || hipEventQuery(se.second) == hipErrorNotReady;
    (void)hipSetDevice(cur);
    if (pending)
        return true;
    p->in_flight = false;
    return false;
}

// ---------------------------------------------------------------------------
// plan cache of ddl_allreduce
// ---------------------------------------------------------------------------
// At most kCacheMax plans are kept; making room destroys the least recently
// used plan that has no work in flight.
constexpr size_t kCacheMax = 64;
struct CacheEntry {
    std::shared_ptr<ddl_plan_s> plan;
    uint64_t used;  // g_cache_tick at the last call
};
// The cache and the registry below are never destroyed: their plans hold
// HIP streams, events and device memory, which must not be released by
// static destructors after the HIP runtime has shut down at process exit.
std::mutex g_cache_mu;
std::map<std::string, CacheEntry> &g_cache = *new std::map<std::string, CacheEntry>;
uint64_t g_cache_tick = 0;

// Destroys least recently used idle plans until fewer than kCacheMax remain
// (or every remaining plan is busy or was captured into a HIP graph, whose
// replays may still read its tables).  Caller holds g_cache_mu, which every
// call on a cached plan also holds, so an idle plan stays idle meanwhile.
void cache_make_room() {
    while (g_cache.size() >= kCacheMax) {
        auto victim = g_cache.end();
        for (auto it = g_cache.begin(); it != g_cache.end(); ++it) {
            if (victim != g_cache.end() && it->second.used >= victim->second.used)
                continue;
            std::lock_guard<std::mutex> pl(it->second.plan->mu);
            if (!it->second.plan->captured && !busy(it->second.plan.get()))
                victim = it;
        }
        if (victim == g_cache.end())
            return;
        g_cache.erase(victim);  // the last reference: the plan is freed
    }
}

// ---------------------------------------------------------------------------
// handles
// ---------------------------------------------------------------------------
// Plans handed to callers (ddl_plan_create, ddl_plan_create_typed) are
// registered here until ddl_plan_destroy; every entry point looks its
// handle up, so a stale or foreign handle is an argument error, not a use
// of freed memory.  The one-shot cache's plans are never handed out and are
// not registered.
void free_plan(ddl_plan_s *p) {
    release_device(p);
    delete p;
}
std::mutex g_live_mu;
std::map<const ddl_plan_s *, std::shared_ptr<ddl_plan_s>> &g_live =
    *new std::map<const ddl_plan_s *, std::shared_ptr<ddl_plan_s>>;

int register_plan(ddl_plan p, ddl_plan *out) {
    std::shared_ptr<ddl_plan_s> sp(p, free_plan);
    std::lock_guard<std::mutex> lk(g_live_mu);
    g_live.emplace(p, std::move(sp));
    *out = p;
    return DDL_OK;
}

// A live plan, its mutex held.  Members are released in reverse order: the
// lock, then the reference (which frees the plan if ddl_plan_destroy let go
// of it meanwhile).
struct PlanRef {
    std::shared_ptr<ddl_plan_s> sp;
    std::unique_lock<std::mutex> lk;
    int rc = DDL_OK;
    ddl_plan_s *operator->() const { return sp.get(); }
    ddl_plan get() const { return sp.get(); }
};

PlanRef acquire(ddl_plan h) {
    PlanRef r;
    if (!h) {
        r.rc = DDL_E_NULL;
        return r;
    }
    {
        std::lock_guard<std::mutex> lk(g_live_mu);
        auto it = g_live.find(h);
        if (it == g_live.end()) {
            r.rc = DDL_E_ARG;
            return r;
        }
        r.sp = it->second;
    }
    r.lk = std::unique_lock<std::mutex>(r.sp->mu);
    if (r.sp->dead) {
        r.lk.unlock();
        r.sp.reset();
        r.rc = DDL_E_ARG;
    }
    return r;
}

void put(std::string &k, const void *p, size_t n) { k.append((const char *)p, n); }

std::string cache_key(int dev, int P, size_t n, int dtype, int op, const ddl_topo &t,
                      const ddl_bucket *buckets, int nb, int mode) {
    std::string k;
    const int hdr[] = {dev, P, dtype, op, t.kind, t.k, t.rows, t.cols, nb, mode,
                       t.ring_order ? 1 : 0};
    put(k, hdr, sizeof(hdr));
    put(k, &n, sizeof(n));
    if (t.ring_order) {
        const size_t cnt = (size_t)(t.kind == DDL_MULTIRING ? std::max(t.k, 0) : 1) * P;
        put(k, t.ring_order, cnt * sizeof(int));
    }
    for (int b = 0; b < nb; ++b) {
        put(k, &buckets[b].offset, sizeof(size_t));
        put(k, &buckets[b].count, sizeof(size_t));
    }
    return k;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

const char *ddl_strerror(int code) {
    switch (code) {
    case DDL_OK: return "ok";
    case DDL_E_NULL: return "a required pointer is NULL";
    case DDL_E_ARG: return "argument out of range (P, n, dtype, op, mode or topology)";
    case DDL_E_BUCKETS: return "buckets do not tile [0, n) exactly";
    case DDL_E_ALIGN: return "a rank buffer is not 16-byte aligned";
    case DDL_E_HIP: return "a HIP runtime call failed";
    case DDL_E_NOMEM: return "allocation failed";
    case DDL_E_BUSY: return "the plan still has work in flight";
    case DDL_E_DEVICE: return "executed on a device other than the plan's";
    case DDL_E_UNBOUND:
        return "the plan has not run on this device yet (its tables are not in device memory)";
    case DDL_E_SCRATCH:
        return "the plan needs more than the allocation-free entry point's fixed scratch";
    default: return "unknown error";
    }
}

}  // extern "C"

namespace {

// A plan for ddl_plan_create and the one-shot cache, not yet registered.
int create_plan(ddl_plan *out, int P, size_t n, ddl_dtype dtype, ddl_op op,
                const ddl_topo *topo, const ddl_bucket *buckets, int nbuckets, ddl_mode mode) {
    if (!out || !topo)
        return DDL_E_NULL;
    *out = nullptr;
    if (mode != DDL_STEPWISE && mode != DDL_FUSED)
        return DDL_E_ARG;
    ddl_plan p = new (std::nothrow) ddl_plan_s;
    if (!p)
        return DDL_E_NOMEM;
    int rc;
    try {
        p->parts.resize(1);
        rc = build_schedule(p->parts[0].s, P, n, dtype, op, *topo, buckets, nbuckets);
        for (int b = 0; !rc && b < (int)p->parts[0].s.buckets.size(); ++b)
            p->order.emplace_back(0, b);
    } catch (const std::bad_alloc &) {
        rc = DDL_E_NOMEM;
    } catch (...) {
        rc = DDL_E_ARG;
    }
    if (rc) {
        delete p;
        return rc;
    }
    p->mode = mode;
    *out = p;
    return DDL_OK;
}

}  // namespace

extern "C" {

int ddl_plan_create(ddl_plan *out, int P, size_t n, ddl_dtype dtype, ddl_op op,
                    const ddl_topo *topo, const ddl_bucket *buckets, int nbuckets,
                    ddl_mode mode) {
    ddl_plan p = nullptr;
    const int rc = create_plan(&p, P, n, dtype, op, topo, buckets, nbuckets, mode);
    if (rc)
        return rc;
    try {
        return register_plan(p, out);
    } catch (...) {
        delete p;
        return DDL_E_NOMEM;
    }
}

int ddl_plan_create_typed(ddl_plan *out, int P, size_t nbytes, ddl_op op, const ddl_topo *topo,
                          const ddl_typed_bucket *buckets, int nbuckets, ddl_mode mode) {
    if (!out || !topo || (nbuckets > 0 && !buckets))
        return DDL_E_NULL;
    *out = nullptr;
    if (mode != DDL_STEPWISE && mode != DDL_FUSED)
        return DDL_E_ARG;
    if (nbuckets < 0 || (nbuckets == 0 && nbytes > 0))
        return DDL_E_BUCKETS;
    // validate in bytes: element-aligned, in range, tiling [0, nbytes)
    std::vector<std::pair<uint64_t, uint64_t>> spans;
    for (int b = 0; b < nbuckets; ++b) {
        const ddl_typed_bucket &t = buckets[b];
        if (t.dtype != DDL_F32 && t.dtype != DDL_F16)
            return DDL_E_ARG;
        const uint64_t esz = t.dtype == DDL_F32 ? 4 : 2;
        if (t.byte_offset % esz || t.byte_offset > nbytes ||
            t.count > (nbytes - t.byte_offset) / esz)
            return DDL_E_BUCKETS;
        if (t.count)
            spans.emplace_back(t.byte_offset, t.count * esz);
    }
    std::sort(spans.begin(), spans.end());
    uint64_t at = 0;
    for (const auto &sp : spans) {
        if (sp.first != at)
            return DDL_E_BUCKETS;
        at += sp.second;
    }
    if (at != nbytes)
        return DDL_E_BUCKETS;
    ddl_plan p = new (std::nothrow) ddl_plan_s;
    if (!p)
        return DDL_E_NOMEM;
    int rc = DDL_OK;
    try {
        // one part per element type present, buckets in list order
        int part_of[2] = {-1, -1};
        std::vector<ddl_bucket> lists[2];
        for (int b = 0; b < nbuckets; ++b) {
            const ddl_typed_bucket &t = buckets[b];
            const uint64_t esz = t.dtype == DDL_F32 ? 4 : 2;
            if (part_of[t.dtype] < 0) {
                part_of[t.dtype] = (int)p->parts.size();
                p->parts.emplace_back();
            }
            p->order.emplace_back(part_of[t.dtype], (int)lists[t.dtype].size());
            lists[t.dtype].push_back({(size_t)(t.byte_offset / esz), t.count, nullptr});
        }
        if (p->parts.empty()) {  // nbytes == 0: an empty binary32 part
            p->parts.emplace_back();
            part_of[DDL_F32] = 0;
        }
        for (int d = 0; d < 2 && !rc; ++d) {
            if (part_of[d] < 0)
                continue;
            const uint64_t esz = d == DDL_F32 ? 4 : 2;
            rc = build_schedule(p->parts[part_of[d]].s, P, nbytes / esz, d, op, *topo,
                                lists[d].data(), (int)lists[d].size(), false);
        }
    } catch (const std::bad_alloc &) {
        rc = DDL_E_NOMEM;
    } catch (...) {
        rc = DDL_E_ARG;
    }
    if (rc) {
        delete p;
        return rc;
    }
    p->typed = true;
    p->mode = mode;
    try {
        return register_plan(p, out);
    } catch (...) {
        delete p;
        return DDL_E_NOMEM;
    }
}

int ddl_plan_execute(ddl_plan plan, void *const *bufs, void *const *ready_events,
                     void *stream, void *done_event) {
    if (!plan || !bufs)
        return DDL_E_NULL;
    try {
        PlanRef r = acquire(plan);
        if (r.rc)
            return r.rc;
        return execute_locked(r.get(), bufs, ready_events, stream, done_event, nullptr);
    } catch (...) {
        return DDL_E_NOMEM;
    }
}

int ddl_plan_execute_sgd(ddl_plan plan, void *const *bufs, void *const *weights, int nweights,
                         float lr, int keep_grads, void *const *ready_events, void *stream,
                         void *done_event) {
    if (!plan || !bufs || !weights)
        return DDL_E_NULL;
    try {
        PlanRef r = acquire(plan);
        if (r.rc)
            return r.rc;
        if (r->typed || (nweights != 1 && nweights != r->parts[0].s.P))
            return DDL_E_ARG;
        if (!keep_grads && r->mode != DDL_FUSED)
            return DDL_E_ARG;
        SgdArgs g;
        std::memset(&g, 0, sizeof(g));
        for (int i = 0; i < nweights; ++i)
            g.w.p[i] = weights[i];
        g.lr = lr;
        g.nweights = nweights;
        g.keep_grads = keep_grads ? 1 : 0;
        return execute_locked(r.get(), bufs, ready_events, stream, done_event, &g);
    } catch (...) {
        return DDL_E_NOMEM;
    }
}

namespace {

// scratch: the allocation-free form, whose partial sums and rates live in
// the library's fixed per-device scratch instead of the plan's buffers.
int execute_lars(ddl_plan plan, void *const *bufs, void *const *weights, int nweights, float lr,
                 double coeff, double eps, float *rates_out, void *const *ready_events,
                 void *stream, void *done_event, bool scratch = false) {
    if (!plan || !bufs || !weights)
        return DDL_E_NULL;
    try {
        PlanRef r = acquire(plan);
        if (r.rc)
            return r.rc;
        if (r->typed || (nweights != 1 && nweights != r->parts[0].s.P))
            return DDL_E_ARG;
        // finite and >= 0 (NaN fails both comparisons)
        if (!(coeff >= 0.0 && coeff <= 1e300) || !(eps >= 0.0 && eps <= 1e300))
            return DDL_E_ARG;
        LarsCall c;
        std::memset(&c, 0, sizeof(c));
        for (int i = 0; i < nweights; ++i)
            c.w.p[i] = weights[i];
        c.nweights = nweights;
        c.lr = lr;
        c.coeff = coeff;
        c.eps = eps;
        c.rates_out = rates_out;
        if (scratch) {
            // sizes first (host-only), then the binding and the device
            const Schedule &s = r->parts[0].s;
            const size_t tiles = lars_tiles(s);
            if (2 * tiles * sizeof(double) > kLarsScratchPartialBytes ||
                s.buckets.size() * sizeof(float) > kLarsScratchBytes - kLarsScratchPartialBytes)
                return DDL_E_SCRATCH;
            if (r->device < 0)
                return DDL_E_UNBOUND;
            int dev = 0;
            if (hipGetDevice(&dev) != hipSuccess)
                return DDL_E_HIP;
            if (dev != r->device)
                return DDL_E_DEVICE;
            void *base = nullptr;
            size_t cap = 0;
            if (lars_scratch(dev, &base, &cap) != hipSuccess || cap < kLarsScratchBytes)
                return DDL_E_HIP;
            c.partial = static_cast<double *>(base);
            c.rate = reinterpret_cast<float *>(static_cast<char *>(base) +
                                               kLarsScratchPartialBytes);
        }
        return execute_locked(r.get(), bufs, ready_events, stream, done_event, nullptr, &c,
                              scratch);
    } catch (...) {
        return DDL_E_NOMEM;
    }
}

}  // namespace

int ddl_plan_execute_lars(ddl_plan plan, void *const *bufs, void *const *weights, int nweights,
                          float lr, double coeff, double eps, float *rates_out,
                          void *const *ready_events, void *stream, void *done_event) {
    return execute_lars(plan, bufs, weights, nweights, lr, coeff, eps, rates_out, ready_events,
                        stream, done_event);
}

int ddl_plan_execute_lars_noalloc(ddl_plan plan, void *const *bufs, void *const *weights,
                                  int nweights, float lr, double coeff, double eps,
                                  float *rates_out, void *const *ready_events, void *stream,
                                  void *done_event) {
    return execute_lars(plan, bufs, weights, nweights, lr, coeff, eps, rates_out, ready_events,
                        stream, done_event, true);
}

int ddl_allreduce(void *const *bufs, int P, size_t n, ddl_dtype dtype, ddl_op op,
                  const ddl_topo *topo, const ddl_bucket *buckets, int nbuckets,
                  ddl_mode mode, void *stream, void *done_event) {
    if (!bufs || !topo || (nbuckets > 0 && !buckets))
        return DDL_E_NULL;
    // the key reads P (or k * P) ring-order entries: range-check them first
    if (P < 1 || P > DDL_MAX_RANKS || (topo->kind == DDL_MULTIRING && topo->k < 1))
        return DDL_E_ARG;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return DDL_E_HIP;
    try {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        const std::string key =
            cache_key(dev, P, n, dtype, op, *topo, buckets, std::max(nbuckets, 0), mode);
        std::shared_ptr<ddl_plan_s> sp;
        auto it = g_cache.find(key);
        if (it != g_cache.end()) {
            sp = it->second.plan;
            it->second.used = ++g_cache_tick;
        } else {
            ddl_plan p = nullptr;
            int rc = create_plan(&p, P, n, dtype, op, topo, buckets, nbuckets, mode);
            if (rc)
                return rc;
            sp = std::shared_ptr<ddl_plan_s>(p, free_plan);
            cache_make_room();
            g_cache.emplace(key, CacheEntry{sp, ++g_cache_tick});
        }
        std::vector<void *> ev(std::max(nbuckets, 0), nullptr);
        for (int b = 0; b < nbuckets; ++b)
            ev[b] = buckets[b].ready_event;
        std::lock_guard<std::mutex> pl(sp->mu);
        return execute_locked(sp.get(), bufs, nbuckets ? ev.data() : nullptr, stream, done_event,
                              nullptr);
    } catch (...) {
        return DDL_E_NOMEM;
    }
}

int ddl_plan_traffic(ddl_plan plan, size_t *sent, size_t *hbm_bytes) {
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    const int P = r->parts[0].s.P;
    size_t hbm = 0;
    for (int i = 0; sent && i < P; ++i)
        sent[i] = 0;
    for (const Part &pt : r->parts) {
        for (int i = 0; sent && i < P; ++i)
            sent[i] += (size_t)pt.s.sent[i];
        hbm += (size_t)(r->mode == DDL_FUSED ? pt.s.fused_bytes : pt.s.step_bytes);
    }
    if (hbm_bytes)
        *hbm_bytes = hbm;
    return DDL_OK;
}

int ddl_plan_destroy(ddl_plan plan) {
    if (!plan)
        return DDL_E_NULL;
    std::shared_ptr<ddl_plan_s> sp;
    {
        std::lock_guard<std::mutex> lk(g_live_mu);
        auto it = g_live.find(plan);
        if (it == g_live.end())
            return DDL_E_ARG;  // never created, or destroyed already
        std::lock_guard<std::mutex> pl(it->second->mu);
        if (busy(it->second.get()))
            return DDL_E_BUSY;
        it->second->dead = true;
        sp = std::move(it->second);
        g_live.erase(it);
    }
    // frees the plan now, or when a call that looked it up before the
    // destroy (and then found it dead) lets go of it
    sp.reset();
    return DDL_OK;
}

int ddl_cache_clear(void) {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    for (auto &kv : g_cache) {
        std::lock_guard<std::mutex> pl(kv.second.plan->mu);
        if (!kv.second.plan->captured && busy(kv.second.plan.get()))
            return DDL_E_BUSY;
    }
    // plans captured into a HIP graph stay: a replay may still read them
    for (auto it = g_cache.begin(); it != g_cache.end();)
        it = it->second.plan->captured ? std::next(it) : g_cache.erase(it);
    return DDL_OK;
}

int ddl_cache_count(size_t *count) {
    if (!count)
        return DDL_E_NULL;
    std::lock_guard<std::mutex> lk(g_cache_mu);
    *count = g_cache.size();
    return DDL_OK;
}

int ddl_plan_set_coalesce_bytes(ddl_plan plan, size_t bytes) {
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    r->coalesce_bytes = bytes;
    return DDL_OK;
}

int ddl_plan_event_groups(ddl_plan plan, int *last, int cap) {
    if (!plan)
        return DDL_E_NULL;
    if (cap < 0 || (cap > 0 && !last))
        return DDL_E_ARG;
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    const int nb = (int)r->order.size();
    int g = 0;
    for (int b0 = 0; b0 < nb; ++g) {
        const int b1 = group_end(r.sp.get(), nullptr, b0, true);
        if (g < cap)
            last[g] = b1 - 1;
        b0 = b1;
    }
    return g;
}

int ddl_plan_set_ordered_events(ddl_plan plan, int ordered) {
    if (!plan)
        return DDL_E_NULL;
    if (ordered != 0 && ordered != 1)
        return DDL_E_ARG;
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    r->ordered_events = ordered != 0;
    return DDL_OK;
}

int ddl_plan_set_side_streams(ddl_plan plan, int n) {
    if (!plan)
        return DDL_E_NULL;
    if (n < 0 || n > kMaxSideStreams)
        return DDL_E_ARG;
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    r->nside = n;
    return DDL_OK;
}

int ddl_plan_set_profiling(ddl_plan plan, int enable) {
    if (!plan)
        return DDL_E_NULL;
    if (enable < 0)
        return DDL_E_ARG;
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    r->profiling = enable != 0;
    r->prof_stride = enable > 1 ? enable : 1;
    r->prof_group = 0;
    return DDL_OK;
}

int ddl_plan_profile_read_kinds(ddl_plan plan, double *total_ms, int *launches,
                                double *max_ms) {
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    ddl_plan_s *const p = r.get();
    double tot[kLaunchKinds] = {}, mx[kLaunchKinds] = {};
    int cnt[kLaunchKinds] = {};
    for (int i = 0; i < p->prof_used; ++i) {
        float ms = 0;
        if (hipEventSynchronize(p->prof[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, p->prof[2 * i], p->prof[2 * i + 1]) != hipSuccess)
            return DDL_E_HIP;
        const int k = p->prof_kind[i];
        tot[k] += ms;
        mx[k] = std::max(mx[k], (double)ms);
        ++cnt[k];
    }
    for (int k = 0; k < kLaunchKinds; ++k) {
        if (total_ms)
            total_ms[k] = tot[k];
        if (launches)
            launches[k] = cnt[k];
        if (max_ms)
            max_ms[k] = mx[k];
    }
    p->prof_used = 0;
    return DDL_OK;
}

int ddl_plan_profile_read(ddl_plan plan, double *total_ms, int *launches, double *max_ms) {
    double tot[kLaunchKinds], mx[kLaunchKinds];
    int cnt[kLaunchKinds];
    const int rc = ddl_plan_profile_read_kinds(plan, tot, cnt, mx);
    if (rc)
        return rc;
    double t = 0, m = 0;
    int c = 0;
    for (int k = 0; k < kLaunchKinds; ++k) {
        t += tot[k];
        c += cnt[k];
        m = std::max(m, mx[k]);
    }
    if (total_ms)
        *total_ms = t;
    if (launches)
        *launches = c;
    if (max_ms)
        *max_ms = m;
    return DDL_OK;
}

int ddl_set_tuning(int knob, int value) {
    if (knob < 0 || knob >= DDL_TUNE_COUNT)
        return DDL_E_ARG;
    g_tune[knob].store(value < 0 ? 0 : (value == INT_MAX ? INT_MAX : value + 1));
    return DDL_OK;
}

int ddl_get_tuning(int knob, int *value) {
    if (!value)
        return DDL_E_NULL;
    if (knob < 0 || knob >= DDL_TUNE_COUNT)
        return DDL_E_ARG;
    *value = tuning(knob);
    return DDL_OK;
}

int ddl_plan_set_fused_passes(ddl_plan plan, int passes) {
    if (!plan)
        return DDL_E_NULL;
    if (passes < 0 || passes > 2)
        return DDL_E_ARG;
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    r->fused_passes = passes;
    return DDL_OK;
}

int ddl_plan_get_fused_passes(ddl_plan plan, int *passes) {
    if (!plan || !passes)
        return DDL_E_NULL;
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    // the form of one group holding all the buckets (of the first element
    // type, for typed plans)
    const Schedule &s = r->parts[0].s;
    uint64_t all = 0;
    for (const Bucket &b : s.buckets)
        all += b.len;
    *passes = r->mode == DDL_FUSED ? fused_passes(r.get(), s, all) : 0;
    return DDL_OK;
}

int ddl_plan_set_step_form(ddl_plan plan, int form) {
    if (!plan)
        return DDL_E_NULL;
    if (form < 0 || form > 2)
        return DDL_E_ARG;
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    r->step_form = form;
    return DDL_OK;
}

int ddl_plan_get_step_form(ddl_plan plan, int *form) {
    if (!plan || !form)
        return DDL_E_NULL;
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    const Schedule &s = r->parts[0].s;
    uint64_t all = 0;
    for (const Bucket &b : s.buckets)
        all += b.len;
    *form = r->mode == DDL_STEPWISE ? step_form(r.get(), s, all) : 0;
    return DDL_OK;
}

int ddl_plan_num_steps(ddl_plan plan, int *steps) {
    if (!plan || !steps)
        return DDL_E_NULL;
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    *steps = r->parts[0].s.nsteps;  // the same for every element type
    return DDL_OK;
}

int ddl_plan_step_kind(ddl_plan plan, int step, int *kind) {
    if (!plan || !kind)
        return DDL_E_NULL;
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    const Schedule &s = r->parts[0].s;
    if (step < 0 || step >= s.nsteps)
        return DDL_E_ARG;
    *kind = s.step_kind[step];
    return DDL_OK;
}

int ddl_plan_step_items(ddl_plan plan, int step, int bucket, ddl_step_item *out, int cap,
                        int *count) {
    if (!plan || !count)
        return DDL_E_NULL;
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    if (bucket < 0 || bucket >= (int)r->order.size())
        return DDL_E_ARG;
    const Schedule &s = r->parts[r->order[bucket].first].s;
    bucket = r->order[bucket].second;
    if (step < 0 || step >= s.nsteps)
        return DDL_E_ARG;
    const uint32_t lo = s.item_at[step][bucket], hi = s.item_at[step][bucket + 1];
    *count = (int)(hi - lo);
    for (uint32_t i = lo; out && i < hi && (int)(i - lo) < cap; ++i) {
        const DevItem &it = s.items[step][i];
        ddl_step_item &o = out[i - lo];
        o.src = it.src;
        o.dst = it.dst;
        o.divide = (it.flags & kItemDivide) ? 1 : 0;
        o.step = step;
        o.offset = (size_t)it.off;
        o.count = (size_t)it.len;
    }
    return DDL_OK;
}

int ddl_plan_fused_spans(ddl_plan plan, int bucket, size_t *offset, size_t *count, int *chain,
                         int cap, int *nspans, int *group) {
    if (!plan || !nspans)
        return DDL_E_NULL;
    PlanRef r = acquire(plan);
    if (r.rc)
        return r.rc;
    if (bucket < 0 || bucket >= (int)r->order.size())
        return DDL_E_ARG;
    const Schedule &s = r->parts[r->order[bucket].first].s;
    bucket = r->order[bucket].second;
    const uint32_t lo = s.span_at[bucket], hi = s.span_at[bucket + 1];
    *nspans = (int)(hi - lo);
    if (group)
        *group = s.group;
    for (uint32_t i = lo; i < hi && (int)(i - lo) < cap; ++i) {
        const DevSpan &sp = s.spans[i];
        if (offset)
            offset[i - lo] = (size_t)sp.off;
        if (count)
            count[i - lo] = (size_t)sp.len;
        if (chain)
            for (int r = 0; r < s.P; ++r)
                chain[(size_t)(i - lo) * s.P + r] = s.chains[sp.chain_off + r];
    }
    return DDL_OK;
}

}  // extern "C"
