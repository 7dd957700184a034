/*
 * ddl.h -- C ABI of libddl.so, the MI355X (gfx950) gradient all-reduce.
 *
 * The operation (Baidu Ring-Allreduce article, part 4, section "总结";
 * Sony "224秒训练ResNet-50" article, the paragraph on synchronising and
 * averaging gradients): P equal-length gradient buffers are summed -- or
 * averaged -- so that every rank ends with the same values.  The all-reduce
 * runs on subsets of the parameters, and the subsets of the output layer go
 * first so that communication overlaps the rest of back-propagation (same
 * Baidu article, its opening paragraphs).  The pages ship the algorithm as a
 * C library that any framework or MPI program can embed (Baidu article,
 * "总结"; IBM DDL blog, last paragraph; "[论文解读] PowerAI DDL", ABSTRACT);
 * this is that library for one GPU that holds the buffers of P virtual ranks.
 *
 * Schedules:
 *  - DDL_RING: ring reduce-scatter then ring all-gather (Baidu article,
 *    "总结" and its reference 4, Patarasuk & Yuan).  Chunk c of a segment
 *    of L elements is piece c of split(L, P, q) (below); in reduce-scatter
 *    step t = 0..P-2 ring position x sends chunk (x-t) mod P to position x+1,
 *    which adds it to its own; in all-gather step t position x sends chunk
 *    (x+1-t) mod P to x+1, which keeps it.
 *  - DDL_MULTIRING: k rings ("[论文解读] PowerAI DDL", ABSTRACT and
 *    "提出的方法"); every bucket is split into k parts by split(L, k, q) and
 *    part j goes round ring j.
 *  - DDL_TORUS2D: rows x cols grid, rank (i, j) = i*cols + j (Sony article,
 *    "2D-Torus All-reduce", Fig. 1 and Fig. 2): ring reduce-scatter along
 *    each row over split(L, cols, q); ring all-reduce down column j over
 *    row-chunk (j+1) mod cols, split into rows sub-chunks; ring all-gather
 *    along each row.
 * split(L, m, q): piece c is [b_c, b_{c+1}), b_c = min(L, q*floor(c*ceil(L/q)/m)),
 * b_m = L, with q = 16 bytes / element size, so every piece of an aligned
 * segment starts on a 16-byte boundary.
 *
 * Arithmetic: DDL_F32 adds in binary32, round to nearest even, subnormals
 * kept.  DDL_F16 stores and exchanges binary16 (Sony article, "训练设置":
 * FP16 gradient exchange): every step computes in binary32 and rounds the
 * result to binary16 (nearest even).  DDL_MEAN divides once by P, correctly
 * rounded, at the add that completes each chunk's sum, before any copy.
 * Results are bit-identical between DDL_STEPWISE and DDL_FUSED, independent
 * of bucket issue order, and identical on every rank.
 *
 * Ownership: the caller owns the buffers (device memory, in place), streams
 * and events.  A plan owns its host and device tables, its side streams and
 * events; it allocates device memory once, on its first execution (the LARS
 * step and two-kernel SGD without kept gradients add a buffer each on their
 * first call), never per call.
 *
 * Errors: every entry point returns DDL_OK (0) or a negative DDL_E_* code;
 * arguments are validated before anything is enqueued, so a failed call
 * enqueues no work.  No C++ exception crosses this interface.
 */
#ifndef DDL_H
#define DDL_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest P a plan accepts (the rank pointers travel as kernel arguments). */
#define DDL_MAX_RANKS 128

typedef enum { DDL_F32 = 0, DDL_F16 = 1 } ddl_dtype;
typedef enum { DDL_SUM = 0, DDL_MEAN = 1 } ddl_op;
typedef enum { DDL_RING = 0, DDL_MULTIRING = 1, DDL_TORUS2D = 2 } ddl_topo_kind;

/* DDL_STEPWISE launches one kernel per schedule step (every pair of every
 * ring, and every bucket of a group, in that one launch).  DDL_FUSED makes
 * one pass per bucket group: each element is read once from every rank,
 * summed in the order the schedule would sum it, and written to every rank. */
typedef enum { DDL_STEPWISE = 0, DDL_FUSED = 1 } ddl_mode;

typedef struct {
    int kind;              /* ddl_topo_kind */
    int k;                 /* DDL_MULTIRING: number of rings (>= 1) */
    int rows, cols;        /* DDL_TORUS2D: rows * cols == P */
    const int *ring_order; /* NULL = identity; else P ints (DDL_RING) or k*P
                              (DDL_MULTIRING): ring j puts rank
                              ring_order[j*P + x] at position x.  Each ring must
                              be a permutation of 0..P-1.  Must be NULL for
                              DDL_TORUS2D.  Copied at plan creation. */
} ddl_topo;

typedef struct {
    size_t offset;         /* first element of the bucket */
    size_t count;          /* elements (0 allowed: nothing to do) */
    void *ready_event;     /* hipEvent_t the bucket waits for, or NULL: ready
                              when the call is made on the caller's stream */
} ddl_bucket;

typedef struct ddl_plan_s *ddl_plan;

enum {
    DDL_OK = 0,
    DDL_E_NULL = -1,     /* a required pointer is NULL */
    DDL_E_ARG = -2,      /* P, n, dtype, op, mode or topology out of range;
                            or a plan handle that no create call returned or
                            that ddl_plan_destroy has freed */
    DDL_E_BUCKETS = -3,  /* buckets do not tile [0, n) exactly */
    DDL_E_ALIGN = -4,    /* a rank buffer is not 16-byte aligned */
    DDL_E_HIP = -5,      /* a HIP runtime call failed */
    DDL_E_NOMEM = -6,    /* host or device allocation failed */
    DDL_E_BUSY = -7,     /* the plan still has work in flight */
    DDL_E_DEVICE = -8,   /* executed on a device other than the plan's */
    DDL_E_UNBOUND = -9,  /* allocation-free call on a plan that has not yet
                            run on the device (ddl_plan_execute_lars_noalloc) */
    DDL_E_SCRATCH = -10  /* the plan needs more than the allocation-free entry
                            point's fixed scratch */
};

/* Build the schedule for P ranks of n elements each.  buckets[0..nbuckets)
 * is the issue order (output layer first for back-propagation overlap) and
 * must tile [0, n) without gap or overlap; their ready_event fields are not
 * used here.  Bucket offsets that are not a multiple of q = 16 B / element
 * size are accepted but run on a slower element-wise path.  Host-only: no
 * HIP call is made, so a plan can be built and inspected without a GPU. */
int ddl_plan_create(ddl_plan *out, int P, size_t n, ddl_dtype dtype, ddl_op op,
                    const ddl_topo *topo, const ddl_bucket *buckets, int nbuckets,
                    ddl_mode mode);

/* A bucket with its own element type, for plans whose buckets do not all
 * share one (some gradients exchanged in binary16, as the Sony ResNet-50
 * article does, others in binary32).  Bucket b covers bytes
 * [byte_offset, byte_offset + count * size(dtype)) of every rank's buffer. */
typedef struct {
    size_t byte_offset;    /* a multiple of the element size */
    size_t count;          /* elements of dtype (0 allowed) */
    ddl_dtype dtype;
} ddl_typed_bucket;

/* Build a plan over P ranks of nbytes bytes each whose buckets carry their
 * own element type.  Each bucket is all-reduced exactly as a plain plan of
 * its dtype would all-reduce it (same chains, same rounding), so the result
 * is bit-identical to one plain plan per dtype.  The buckets must tile
 * [0, nbytes) in bytes without gap or overlap (DDL_E_BUCKETS), and each
 * byte_offset must be a multiple of its element size (DDL_E_BUCKETS); list
 * order is issue order.  Run it with ddl_plan_execute (ready_events, if
 * given, one per typed bucket in list order); consecutive buckets with equal
 * events form a group, as in plain plans, and a group runs one pass (or one
 * step sequence) per dtype it holds.
 * ddl_plan_execute_sgd returns DDL_E_ARG for such a plan (its weights are
 * indexed by element, which typed buckets do not define), and
 * ddl_plan_traffic's per-rank counts add up elements of both types.
 * Introspection calls take typed bucket indices.  Host-only, like
 * ddl_plan_create. */
int ddl_plan_create_typed(ddl_plan *out, int P, size_t nbytes, ddl_op op,
                          const ddl_topo *topo, const ddl_typed_bucket *buckets, int nbuckets,
                          ddl_mode mode);

/* Enqueue the all-reduce of bufs[0..P) (device pointers, each 16-byte
 * aligned, n elements) on the current HIP device.
 *  ready_events  NULL, or nbuckets hipEvent_t (entries may be NULL) in bucket
 *                list order: bucket b's work waits for ready_events[b].  The
 *                library only makes its streams wait for them and never
 *                inspects them from the host, so events created with
 *                hipEventDisableSystemFence serve: their records skip the
 *                cache writeback and invalidate of the default fence.
 *  stream        the caller's hipStream_t (NULL = default stream).  Buckets
 *                without an event wait for the work already enqueued on it.
 *  done_event    NULL or a hipEvent_t recorded when every bucket is done.
 * Buckets with events run on the plan's side stream, in list order; the
 * caller's stream is made to wait for the whole all-reduce before its next
 * work.  Asynchronous: returns after enqueueing; do not touch bufs until
 * done_event completes or the stream is synchronised.  The first call on a
 * plan uploads its tables (a synchronous copy, once).  Concurrent calls on
 * one plan are serialised by a mutex; calls on different plans that share
 * buffers race. */
int ddl_plan_execute(ddl_plan plan, void *const *bufs, void *const *ready_events,
                     void *stream, void *done_event);
/* HIP graph capture: every execute entry point may be captured on the
 * caller's stream once the plan has run eagerly on the device (its first
 * call allocates and uploads its tables, as does the first LARS call and
 * the first two-kernel SGD call without kept gradients).  The graph then
 * holds the plan's table addresses: see ddl_plan_destroy. */

/* The all-reduce followed by the SGD step it serves, fused into the
 * reduction's epilogue (the Baidu article, "总结": the all-reduce averages
 * gradients for synchronous stochastic gradient descent).  Once the reduced
 * gradient y reaches a rank, that rank's binary32 weights take
 *     w[e] = w[e] - lr * y[e]
 * (binary16 y widened exactly; the product rounded before the difference).
 *  weights     nweights device pointers to n binary32 elements, 16-byte
 *              aligned: nweights == P gives one replica per rank (each
 *              updated once), nweights == 1 one replica shared by all ranks
 *              (updated once).  Replicas must not overlap each other or bufs.
 *  keep_grads  1: bufs end with the all-reduce result as ddl_plan_execute
 *              leaves them.  0 (DDL_FUSED plans only): bufs are left as they
 *              were -- the reduced gradient is consumed by the update and
 *              never written, saving P writes per element.
 * In DDL_FUSED plans the update rides in the one-kernel pass's epilogue, or
 * follows the two-kernel pass (ddl_plan_set_fused_passes).  In DDL_STEPWISE
 * plans, in either step form, the owner of each chunk updates at the add that
 * completes the sum and every other rank when the all-gather delivers it.
 * Other arguments and the asynchrony are those of ddl_plan_execute.  Calls
 * with keep_grads == 0 in the two-kernel form share the plan's scratch
 * buffer: two such calls on one plan that may run at the same time on the
 * device race; order them.
 * DDL_E_ARG for any other nweights, or keep_grads == 0 on a stepwise plan. */
int ddl_plan_execute_sgd(ddl_plan plan, void *const *bufs, void *const *weights, int nweights,
                         float lr, int keep_grads, void *const *ready_events, void *stream,
                         void *done_event);

/* The all-reduce followed by a LARS step (Sony ResNet-50 article, "训练设置":
 * the weights are updated with LARS, coefficient 0.01 and eps 1e-6; the
 * page omits the formula, taken here from You, Gitman and Ginsburg's
 * layer-wise adaptive rate scaling without weight decay or momentum).  Each
 * bucket is a layer.  Once the bucket is all-reduced (bufs end with the
 * result, as after ddl_plan_execute), from replica 0's weights w and the
 * reduced gradient y over the bucket:
 *     trust = coeff * ||w|| / (||y|| + eps)   (1 if ||w|| or ||y|| is 0)
 *     rate  = binary32(lr * trust)            (norms and trust in binary64)
 * and every replica takes w[e] = w[e] - rate * y[e] as in
 * ddl_plan_execute_sgd.  Replicas of a synchronous step are identical, so
 * replica 0's norm serves all of them.
 *  weights     as for ddl_plan_execute_sgd (nweights 1 or P).
 *  coeff, eps  the trust coefficient and eps (the page: 0.01 and 1e-6);
 *              finite and >= 0, else DDL_E_ARG.
 *  rates_out   NULL, or device memory for nbuckets binary32 values that
 *              receive each bucket's rate (bucket list order).
 * The norms are sums of squares in binary64, deterministic but not in index
 * order, so a rate can differ from an index-order evaluation when lr * trust
 * lies within about 1e-13 (relative) of a binary32 rounding boundary.  The
 * first call allocates 16 bytes per tile of the plan's buckets (a tile is
 * 4 KB: 1024 binary32 or 2048 binary16 elements) plus 4 per bucket, once.
 * The partial sums and rates are the plan's: two LARS calls on one plan that
 * may run at the same time on the device (different streams, no ordering
 * event) race; order them.
 * DDL_E_ARG for a plan with typed buckets or another nweights.  Other
 * arguments and the asynchrony are those of ddl_plan_execute. */
int ddl_plan_execute_lars(ddl_plan plan, void *const *bufs, void *const *weights, int nweights,
                          float lr, double coeff, double eps, float *rates_out,
                          void *const *ready_events, void *stream, void *done_event);

/* The LARS step of ddl_plan_execute_lars for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same all-reduce and the same LARS arithmetic,
 * bit for bit, but the per-tile partial sums and per-bucket rates live in
 * a fixed scratch array the library holds on every device it runs on
 * (8 MiB of partial sums, 16 bytes per 4 KB tile -- at most 524,288 tiles
 * over the plan's buckets, 536,870,912 binary32 elements in whole tiles --
 * and 256 KiB of rates, at most 65,536 buckets), instead of the buffers
 * ddl_plan_execute_lars allocates on its first call.  This call makes no
 * device allocation and creates no HIP stream or event: the plan must
 * already have run on the current device (any execute entry point binds it;
 * otherwise DDL_E_UNBOUND), and profiling brackets are not recorded.
 * DDL_E_SCRATCH, before anything else, for a plan whose tiles or buckets
 * exceed the scratch; DDL_E_NOMEM if the plan has already run on eight
 * other streams and this one is new (its completion tracking would need a
 * new event; reported before anything is enqueued).  The scratch keeps the last call's contents and every call on
 * a device shares it: two such calls that may run at the same time on one
 * device (any plans, different streams, no ordering between them) race.
 * Other arguments, errors and the asynchrony are those of
 * ddl_plan_execute_lars. */
int ddl_plan_execute_lars_noalloc(ddl_plan plan, void *const *bufs, void *const *weights,
                                  int nweights, float lr, double coeff, double eps,
                                  float *rates_out, void *const *ready_events, void *stream,
                                  void *done_event);

/* One-shot form: looks up (or builds and caches) the plan for these
 * arguments -- the cache key is everything except the buffers and events --
 * and executes it with the buckets' ready_event fields.  Thread-safe.  The
 * cache holds at most 64 plans: a new one first destroys the least recently
 * used plan that has no work in flight and was never captured into a HIP
 * graph (freeing its device tables, which waits for the device like any
 * hipFree). */
int ddl_allreduce(void *const *bufs, int P, size_t n, ddl_dtype dtype, ddl_op op,
                  const ddl_topo *topo, const ddl_bucket *buckets, int nbuckets,
                  ddl_mode mode, void *stream, void *done_event);

/* Traffic of the schedule.  sent_elems_per_rank (NULL or P entries): the
 * elements each rank sends over the whole schedule, 2 (P-1)/P * n for a ring
 * when P*q divides every bucket (Patarasuk & Yuan's bandwidth-optimal
 * count; the Baidu article's "1.2 GB gradient -> about 2.4 GB sent and
 * received").  hbm_bytes (NULL allowed): the algorithmic bytes the plan's
 * kernels read plus write per execution -- 2 P n s for DDL_FUSED (every
 * rank's input read once, its result written once; the two-kernel form
 * re-reads the n s bytes of results from the device caches on top, which
 * this count leaves out), 5 (P-1) n s for DDL_STEPWISE (3 L s per
 * reduce-scatter step, 2 L s per all-gather step). */
int ddl_plan_traffic(ddl_plan plan, size_t *sent_elems_per_rank, size_t *hbm_bytes);

/* Free the plan.  Returns DDL_E_BUSY, and frees nothing, while work the plan
 * enqueued has not completed; DDL_E_ARG for a handle that is not a live plan
 * (destroyed already, or never created), which is checked against the
 * library's registry of live plans before anything is touched, so a second
 * destroy or a call on a destroyed handle is an error code, not a use of freed
 * memory.
 * HIP graphs: an execution captured into a HIP graph (see ddl_plan_execute)
 * keeps the addresses of the plan's device tables in the graph, and the
 * library cannot see the graph's replays.  A plan must outlive every graph
 * and graph executable made from a capture of it: destroy those first. */
int ddl_plan_destroy(ddl_plan plan);

/* Drop every plan ddl_allreduce cached (DDL_E_BUSY if one is in flight).
 * Plans whose execution was captured into a HIP graph stay cached until the
 * process ends: a replay of the graph may still read them. */
int ddl_cache_clear(void);

/* Number of plans ddl_allreduce holds in its cache. */
int ddl_cache_count(size_t *count);

/* Static text for a DDL_* code. */
const char *ddl_strerror(int code);

/* ---- merging of ready buckets ------------------------------------------ *
 * IBM's multi-ring trades latency against bandwidth ("[论文解读] PowerAI
 * DDL", ABSTRACT).  At execution consecutive buckets (in list order) whose
 * ready events are equal -- NULL included -- always share one group of
 * launches.  With a threshold > 0, a group also absorbs following buckets
 * with other events until it holds that many bytes per rank; it then waits
 * for all their events before it starts.  Default 0. */
int ddl_plan_set_coalesce_bytes(ddl_plan plan, size_t bytes);

/* The groups a call forms, at the current threshold, when every bucket has a
 * ready event of its own: returns their number G (>= 1 for a plan with
 * buckets; a negative DDL_E_* code on error) and writes to last[g], for
 * g < min(G, cap), the list index of group g's last bucket (increasing; the
 * last is nbuckets - 1).  A caller that records one ready event per group
 * -- once the gradients of buckets last[g-1]+1 .. last[g] are complete --
 * and passes it for each of those buckets gets the same groups and the same
 * results, with one event record and one wait per group instead of one per
 * bucket: each record costs the device a few microseconds, more than a
 * small bucket's share of the pass.  last may be NULL with cap = 0 to count
 * only; DDL_E_ARG for cap < 0 or a NULL last with cap > 0. */
int ddl_plan_event_groups(ddl_plan plan, int *last, int cap);

/* The caller's promise that it records the buckets' ready events in list
 * order on one stream -- as back-propagation produces the gradients, output
 * layer first (Baidu article, opening paragraphs) -- so that the completion
 * of bucket b's event implies that of every earlier bucket's.  With
 * ordered = 1 a group of buckets (coalesced up to ddl_plan_set_coalesce_bytes)
 * waits only for the event of its last bucket that has one, instead of one
 * wait per distinct event: each wait costs the device a few microseconds.
 * Buckets without an event still wait for the caller's stream as of the
 * call.  If the promise does not hold, a bucket may be reduced before its
 * gradient is complete.  Default 0; DDL_E_ARG for values other than 0, 1. */
int ddl_plan_set_ordered_events(ddl_plan plan, int ordered);

/* Event-gated groups alternate over n side streams (1..4) in list order.
 * Buckets are independent all-reduces, so a group's kernels may run while
 * the previous group's drain; the results do not change.  n = 0 (default):
 * automatic, 2 for stepwise plans and for fused plans whose buckets average
 * under 4 MB per rank (short launches whose ramps overlap), else 1. */
int ddl_plan_set_side_streams(ddl_plan plan, int n);

/* Form of a fused plan's pass (fused mode only).  passes = 1: one kernel
 * reads every rank and writes every rank (with the SGD step, it also updates
 * the weights).  passes = 2: a reduce kernel reads every rank and writes the
 * result to rank 0, then a broadcast kernel copies it from rank 0 to ranks
 * 1..P-1 while it is still in the device caches, so HBM serves a read phase
 * and then a write phase; with the SGD step the broadcast also steps the
 * weights as it copies (without kept gradients the reduce kernel writes to a
 * scratch buffer of n elements instead, allocated by the first such call,
 * nothing is broadcast, and an update kernel steps the weights from it).  passes = 0 (default): automatic,
 * per group: two kernels from 16 ranks on for groups of at least 200 MB
 * summed over the ranks (400 MB for binary16), one kernel otherwise (short
 * passes are launch-bound, and the second launch costs more than it saves).
 * The results are bit-identical either way; only the speed differs.
 * Returns DDL_E_ARG for other values.  Takes effect at the next execute.
 * ddl_plan_get_fused_passes reports the form of one group holding all the
 * plan's buckets, as in a call without ready events (0 for a stepwise
 * plan). */
int ddl_plan_set_fused_passes(ddl_plan plan, int passes);
int ddl_plan_get_fused_passes(ddl_plan plan, int *passes);

/* Form of a stepwise plan's execution (stepwise mode only).
 * form = 1: one kernel launch per schedule step, every pair of the step in
 * that launch.  form = 2: one persistent launch per group of buckets.  Every
 * dependency of the schedule is per element (a step reads element e of a
 * rank only where an earlier step wrote element e), so each workgroup takes
 * one tile of a chunk (torus: of a sub-chunk) and carries it through every
 * reduce-scatter and all-gather step in schedule order, reading and writing
 * the ranks' buffers at each step as the per-step launches do (the same
 * bytes, the same results); no barrier spans workgroups.  This is the
 * latency form for small buckets ("[论文解读] PowerAI DDL", ABSTRACT: the
 * latency/bandwidth trade-off): 2 (P-1) launches become one.
 * form = 0 (default): automatic, which is the persistent form (measured the
 * faster on every workload).  The SGD step (ddl_plan_execute_sgd) rides on
 * either form.
 * DDL_E_ARG for other values; takes effect at the next execute.
 * ddl_plan_get_step_form reports the form of one group holding all the
 * plan's buckets, as in a call without ready events (0 for a fused plan). */
int ddl_plan_set_step_form(ddl_plan plan, int form);
int ddl_plan_get_step_form(ddl_plan plan, int *form);

/* ---- tuning ------------------------------------------------------------ *
 * Process-wide knobs of the fused pass's kernels, for benchmarks.  They
 * change speed only, never results, and take effect at the next launch.
 * ddl_set_tuning with a negative value restores the default; both return
 * DDL_E_ARG for an unknown knob. */
typedef enum {
    /* two-kernel form: ranks each broadcast workgroup writes; 0 = automatic
     * (2 from 32 ranks on, 7 below) */
    DDL_TUNE_BCAST_RANKS = 0,
    /* two-kernel form: 1 = the reduce kernel's loads are non-temporal
     * (default), 0 = cached */
    DDL_TUNE_REDUCE_NT_LOAD = 1,
    /* one-kernel form: loads are non-temporal while P x the elements a lane
     * loads per rank is at most 4 x this (default 24: up to 24 binary32
     * ranks, 12 binary16 ranks) */
    DDL_TUNE_FUSED_NT_LOAD_MAX_P = 2,
    /* tile anchoring of the plans created afterwards: 0 = automatic (tables
     * whose ranges average at least 2 tiles), 1 = never, 2 = always */
    DDL_TUNE_ANCHOR = 3,
    /* loads each lane issues ahead of their adds (1, 2, 4 or 8; other values
     * act as 1) in the one-kernel pass (default 1) and in the reduce
     * kernel's tile-by-tile form (default 4); the adds keep the schedule's
     * order */
    DDL_TUNE_FUSED_BATCH = 4,
    DDL_TUNE_REDUCE_BATCH = 5,
    /* two-kernel form: consecutive tiles each broadcast workgroup copies
     * (default 1; at most 64) */
    DDL_TUNE_BCAST_TILES = 6,
    /* two-kernel form: deal the broadcast's workgroups so that all rank
     * groups of a tile run on one of this many accelerator dies (8 on
     * MI355X), which fetches the tile's values into that die's L2 once;
     * 0 or 1 = plain order (default) */
    DDL_TUNE_BCAST_XCD = 7,
    /* update kernel (the LARS step, and the SGD step of the two-kernel
     * form): weight replicas each workgroup steps (default 2); 0 = all of
     * them in one workgroup */
    DDL_TUNE_UPDATE_REPS = 8,
    /* update kernel, and the broadcast that updates the replicas in the
     * LARS step's two-kernel form: replicas whose loads each lane issues
     * before their stores (1, 2, 4 or 8; default 4; the broadcast takes 8
     * as 4) */
    DDL_TUNE_UPDATE_BATCH = 9,
    /* two-kernel form: the reduce kernel walks the tiles of each workgroup
     * rank by rank (six tiles per workgroup from 32 ranks on, four below;
     * the loads of one rank two at a time) from this many ranks on, and
     * tile by tile (one tile per workgroup, DDL_TUNE_REDUCE_BATCH loads at a
     * time) below; default 16 */
    DDL_TUNE_REDUCE_RANKS_MIN_P = 10,
    /* two-kernel form: the broadcast waits for each rank's stores to
     * complete before storing to the next rank (and, in the broadcast that
     * steps weight replicas, for each batch of replicas): 0 never, 1
     * always, 2 (default) for binary32 */
    DDL_TUNE_BCAST_STORE_WAIT = 11,
    /* one-kernel form: each workgroup waits for each rank's stores to
     * complete before storing to the next rank: 0 never, 1 always, 2
     * (default) for binary32 groups of at least 2^27 elements per rank from
     * 8 ranks on */
    DDL_TUNE_FUSED_STORE_WAIT = 12,
    DDL_TUNE_COUNT = 13
} ddl_tune_knob;
int ddl_set_tuning(int knob, int value);
int ddl_get_tuning(int knob, int *value);

/* ---- measurement -------------------------------------------------------- *
 * With profiling on, kernel launches are bracketed by a pair of HIP events
 * on the stream they are launched on: enable = 1 brackets every launch;
 * enable = m > 1 brackets the launches of every m-th group of buckets (the
 * groups counted across calls from this setting on), so that a timed run is
 * barely slowed; 0 turns it off; negative values are DDL_E_ARG.
 * ddl_plan_profile_read waits for the last of them and reports, for all
 * bracketed launches since the previous read, the sum of their durations
 * (ms), their number and the longest one; then it starts a new count.
 * Costs a few microseconds per bracketed launch. */
int ddl_plan_set_profiling(ddl_plan plan, int enable);
int ddl_plan_profile_read(ddl_plan plan, double *total_ms, int *launches, double *max_ms);
/* The same, per launch kind: each argument (or NULL) is an array of
 * DDL_K_COUNT entries indexed by ddl_launch_kind. */
int ddl_plan_profile_read_kinds(ddl_plan plan, double *total_ms, int *launches,
                                double *max_ms);

/* ---- schedule introspection (host-only; used by the tests) ------------- */
/* Kernel launches: a reduce-scatter step, an all-gather step, the one-kernel
 * fused pass, the two kernels of the two-kernel fused pass, the LARS step's
 * norms and rates, the weight update (of the LARS step, and of the SGD step
 * in the two-kernel form), and the persistent step kernel of a stepwise
 * group (ddl_plan_set_step_form). */
typedef enum {
    DDL_K_REDUCE = 0,
    DDL_K_GATHER = 1,
    DDL_K_FUSED = 2,
    DDL_K_FUSED_REDUCE = 3,
    DDL_K_BROADCAST = 4,
    DDL_K_LARS_NORM = 5,
    DDL_K_LARS_RATE = 6,
    DDL_K_UPDATE = 7,
    DDL_K_WALK = 8,
    DDL_K_COUNT = 9
} ddl_launch_kind;

/* One pair transfer of one step: rank dst combines elements
 * [offset, offset+count) of rank src into its own (DDL_K_REDUCE, dividing
 * by P afterwards when divide is set) or copies them (DDL_K_GATHER). */
typedef struct {
    int src, dst, divide, step;
    size_t offset, count;
} ddl_step_item;

/* Number of schedule steps of one bucket (2(P-1) ring and multi-ring,
 * 2(rows-1) + 2(cols-1) torus) and the kind of step s. */
int ddl_plan_num_steps(ddl_plan plan, int *steps);
int ddl_plan_step_kind(ddl_plan plan, int step, int *kind);
/* The items of step `step` for bucket `bucket` (list index).  *count gets the
 * number of items; up to cap of them are written to out (out may be NULL). */
int ddl_plan_step_items(ddl_plan plan, int step, int bucket, ddl_step_item *out,
                        int cap, int *count);
/* The fused spans of bucket `bucket`: span i covers [offset[i], offset[i]+
 * count[i]) and sums ranks chain[i*P .. i*P+P-1] in that order, in groups
 * of `group` consecutive entries (group = P for rings, cols for the torus):
 * each group left to right, then the group sums left to right. */
int ddl_plan_fused_spans(ddl_plan plan, int bucket, size_t *offset, size_t *count,
                         int *chain, int cap, int *nspans, int *group);

#ifdef __cplusplus
}
#endif
#endif
