// plan_asan_driver.cpp -- host-only driver of the plan layer (plan.cpp and
// schedule.cpp), built by the test suite with AddressSanitizer and
// UndefinedBehaviorSanitizer (g++, no GPU code).
//
// The HIP runtime calls the plan layer makes are replaced here by a fake
// device: device memory is host memory, streams and events are tokens, every
// call succeeds.  The kernel launchers are replaced by checks of their
// arguments (tile ranges inside the tables they index).  Random plain and
// typed plans then run every entry point -- execute in both modes and both
// fused forms, with and without ready events, side streams and coalescing,
// the SGD and LARS steps, introspection, the one-shot form through its
// bounded cache, busy tracking, destroy -- so that any out-of-bounds access,
// leak-prone path or undefined behaviour in the host code is reported.
// Exit status 0 and "ok N cases" when everything holds.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "../sgd_gradient_all_amd/csrc/ddl_internal.h"

// ---------------------------------------------------------------------------
// fake device
// ---------------------------------------------------------------------------
static long g_live_allocs = 0, g_live_streams = 0, g_live_events = 0;

extern "C" {
hipError_t hipMalloc(void **p, size_t n) {
    *p = std::malloc(n ? n : 1);
    ++g_live_allocs;
    return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void *p) {
    if (p) {
        std::free(p);
        --g_live_allocs;
    }
    return hipSuccess;
}
hipError_t hipMemcpy(void *d, const void *s, size_t n, hipMemcpyKind) {
    std::memcpy(d, s, n);
    return hipSuccess;
}
hipError_t hipGetDevice(int *d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipStreamCreateWithFlags(hipStream_t *s, unsigned) {
    *s = reinterpret_cast<hipStream_t>(new int(1));
    ++g_live_streams;
    return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t s) {
    delete reinterpret_cast<int *>(s);
    --g_live_streams;
    return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t *e) {
    *e = reinterpret_cast<hipEvent_t>(new int(2));
    ++g_live_events;
    return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t *e, unsigned) { return hipEventCreate(e); }
hipError_t hipEventDestroy(hipEvent_t e) {
    delete reinterpret_cast<int *>(e);
    --g_live_events;
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) {
    return *reinterpret_cast<int *>(e) == 2 ? hipSuccess : hipErrorInvalidValue;
}
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t e, unsigned) {
    // caller events are tokens of this driver too (value 2)
    return *reinterpret_cast<int *>(e) == 2 ? hipSuccess : hipErrorInvalidValue;
}
hipError_t hipEventQuery(hipEvent_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float *ms, hipEvent_t, hipEvent_t) {
    *ms = 0.f;
    return hipSuccess;
}
}

// ---------------------------------------------------------------------------
// launchers: argument checks instead of kernels
// ---------------------------------------------------------------------------
static long g_launches = 0;
static void fail(const char *what) {
    std::printf("FAILED: %s\n", what);
    std::exit(1);
}
namespace ddl {
int launch_step(int, int, int vpl, const RankPtrs &, const StepArgs &a, const SgdArgs *,
                uint32_t tiles, void *) {
    if (!a.items || !a.prefix || tiles == 0 || (vpl != 1 && vpl != 2 && vpl != 4))
        fail("step launch arguments");
    if (a.prefix[a.item_lo] > a.tile_base || a.tile_base + tiles > a.prefix[a.item_hi])
        fail("step launch tiles outside the step's items");
    ++g_launches;
    return 0;
}
int launch_fused(int, const RankPtrs &, const FusedArgs &a, const SgdArgs *, bool home,
                 uint32_t tiles, void *) {
    if (!a.spans || !a.prefix || !a.tile_span || !a.chains || tiles == 0 ||
        a.tile_end - a.tile_base != tiles || (home && !a.home))
        fail("fused launch arguments");
    if (a.prefix[a.span_lo] > a.tile_base || a.tile_end > a.prefix[a.span_hi])
        fail("fused launch tiles outside the group's spans");
    for (uint32_t t = a.tile_base; t < a.tile_end; t += 97) {
        const uint32_t i = a.tile_span[t];
        if (i < a.span_lo || i >= a.span_hi || a.prefix[i] > t || t >= a.prefix[i + 1])
            fail("tile -> span table");
    }
    ++g_launches;
    return 0;
}
int launch_bcast(int, const RankPtrs &, const BcastArgs &a, void *) {
    if (a.ranks_per_group < 1 || a.ngroups < 1 || a.tiles_per_group < 1 ||
        1 + (a.ngroups - 1) * a.ranks_per_group >= a.P)
        fail("broadcast launch arguments");
    if (a.spans && (a.tile_end <= a.tile_base || !a.prefix || !a.tile_span))
        fail("broadcast table launch");
    if (!a.spans && a.len == 0)
        fail("empty broadcast run");
    ++g_launches;
    return 0;
}
int launch_tiny(int, const RankPtrs &, const TinyArgs &a, void *) {
    if (!a.spans || !a.tiny || !a.chains || a.hi <= a.lo)
        fail("tiny launch arguments");
    for (uint32_t t = a.lo; t < a.hi; ++t)
        if (a.spans[a.tiny[t]].len > kTinySpanMax || a.spans[a.tiny[t]].len == 0)
            fail("tiny span length");
    ++g_launches;
    return 0;
}
int launch_lars(int, int, const RankPtrs &, const LarsArgs &a, uint32_t blocks, void *) {
    if (blocks == 0 || !a.spans || !a.prefix)
        fail("LARS launch arguments");
    ++g_launches;
    return 0;
}
}  // namespace ddl

// ---------------------------------------------------------------------------
// random cases
// ---------------------------------------------------------------------------
static int check(int rc, const char *what) {
    if (rc != DDL_OK) {
        std::printf("FAILED: %s returned %d (%s)\n", what, rc, ddl_strerror(rc));
        std::exit(1);
    }
    return rc;
}

int main(int argc, char **argv) {
    const int ncases = argc > 1 ? std::atoi(argv[1]) : 200;
    std::mt19937_64 rng(12345);
    auto uni = [&](int lo, int hi) { return lo + (int)(rng() % (uint64_t)(hi - lo + 1)); };
    for (int c = 0; c < ncases; ++c) {
        const int Ps[] = {1, 2, 3, 5, 8, 16, 40, 128};
        const int P = Ps[uni(0, 7)];
        ddl_topo topo = {DDL_RING, 1, 0, 0, nullptr};
        const int kind = uni(0, 2);
        if (kind == 1) {
            topo.kind = DDL_MULTIRING;
            topo.k = uni(1, 5);
        } else if (kind == 2) {
            std::vector<int> divs;
            for (int r = 1; r <= P; ++r)
                if (P % r == 0)
                    divs.push_back(r);
            topo.kind = DDL_TORUS2D;
            topo.rows = divs[uni(0, (int)divs.size() - 1)];
            topo.cols = P / topo.rows;
        }
        const int nb = uni(1, 12);
        std::vector<ddl_bucket> bk(nb);
        size_t n = 0;
        for (int b = 0; b < nb; ++b) {
            const int r = uni(0, 9);
            const size_t cnt = r == 0 ? 0 : r < 4 ? uni(1, 200) : r < 8 ? uni(200, 30000)
                                                                         : uni(30000, 300000);
            bk[b] = {n, cnt, nullptr};
            n += cnt;
        }
        std::shuffle(bk.begin(), bk.end(), rng);
        const ddl_dtype dt = uni(0, 1) ? DDL_F16 : DDL_F32;
        const ddl_op op = uni(0, 1) ? DDL_MEAN : DDL_SUM;
        const ddl_mode mode = uni(0, 1) ? DDL_FUSED : DDL_STEPWISE;
        ddl_plan plan = nullptr;
        check(ddl_plan_create(&plan, P, n, dt, op, &topo, bk.data(), nb, mode), "create");
        // fake device buffers: 16-byte aligned host memory
        const size_t esz = dt == DDL_F32 ? 4 : 2;
        std::vector<void *> bufs(P), w(P);
        for (int r = 0; r < P; ++r) {
            bufs[r] = std::aligned_alloc(16, ((n * esz + 15) / 16 + 1) * 16);
            w[r] = std::aligned_alloc(16, ((n * 4 + 15) / 16 + 1) * 16);
        }
        std::vector<hipEvent_t> ev(nb);
        std::vector<void *> evp(nb);
        for (int b = 0; b < nb; ++b) {
            (void)hipEventCreate(&ev[b]);
            evp[b] = (b % 3 == 2) ? nullptr : ev[b - b % 2];
        }
        hipStream_t s;
        (void)hipStreamCreateWithFlags(&s, 0);
        check(ddl_plan_set_side_streams(plan, uni(0, 4)), "side streams");
        check(ddl_plan_set_coalesce_bytes(plan, uni(0, 1) ? 0 : (size_t)uni(1, 1 << 22)),
              "coalesce");
        if (mode == DDL_FUSED)
            check(ddl_plan_set_fused_passes(plan, uni(0, 2)), "passes");
        check(ddl_plan_set_profiling(plan, uni(0, 1)), "profiling");
        for (int rep = 0; rep < 2; ++rep) {
            check(ddl_plan_execute(plan, bufs.data(), uni(0, 1) ? evp.data() : nullptr, s, ev[0]),
                  "execute");
            check(ddl_plan_execute_sgd(plan, bufs.data(), w.data(), uni(0, 1) ? 1 : P, 0.01f, 1,
                                       evp.data(), s, nullptr),
                  "execute_sgd");
            if (mode == DDL_FUSED)
                check(ddl_plan_execute_sgd(plan, bufs.data(), w.data(), P, 0.01f, 0, nullptr, s,
                                           nullptr),
                      "execute_sgd without kept gradients");
            check(ddl_plan_execute_lars(plan, bufs.data(), w.data(), uni(0, 1) ? 1 : P, 0.01f,
                                        0.01, 1e-6, nullptr, uni(0, 1) ? evp.data() : nullptr,
                                        s, nullptr),
                  "execute_lars");
        }
        double tot[DDL_K_COUNT], mx[DDL_K_COUNT];
        int cnt[DDL_K_COUNT];
        check(ddl_plan_profile_read_kinds(plan, tot, cnt, mx), "profile read");
        std::vector<size_t> sent(P);
        size_t hbm = 0;
        check(ddl_plan_traffic(plan, sent.data(), &hbm), "traffic");
        int steps = 0;
        check(ddl_plan_num_steps(plan, &steps), "num_steps");
        for (int st = 0; st < steps; st += 3) {
            int k = 0, m = 0;
            check(ddl_plan_step_kind(plan, st, &k), "step_kind");
            check(ddl_plan_step_items(plan, st, 0, nullptr, 0, &m), "step_items count");
            std::vector<ddl_step_item> items(m + 1);
            check(ddl_plan_step_items(plan, st, 0, items.data(), m, &m), "step_items");
        }
        check(ddl_plan_destroy(plan), "destroy");
        // the one-shot form and its bounded cache
        ddl_bucket whole = {0, n, nullptr};
        check(ddl_allreduce(bufs.data(), P, n, dt, op, &topo, n ? &whole : nullptr, n ? 1 : 0,
                            mode, s, nullptr),
              "ddl_allreduce");
        size_t cached = 0;
        check(ddl_cache_count(&cached), "cache count");
        if (cached > 64)
            fail("cache above its bound");
        for (int b = 0; b < nb; ++b)
            (void)hipEventDestroy(ev[b]);
        (void)hipStreamDestroy(s);
        for (int r = 0; r < P; ++r) {
            std::free(bufs[r]);
            std::free(w[r]);
        }
        // a typed plan over a random mixed layout
        std::vector<ddl_typed_bucket> tb;
        size_t at = 0;
        const int ntb = uni(1, 10);
        for (int b = 0; b < ntb; ++b) {
            const ddl_dtype d = uni(0, 1) ? DDL_F16 : DDL_F32;
            const size_t e = d == DDL_F32 ? 4 : 2;
            if (at % e) {
                tb.back().count += 1;
                at += 2;
            }
            const size_t cnt = uni(0, 3) == 0 ? 0 : uni(1, 5000);
            tb.push_back({at, cnt, d});
            at += cnt * e;
        }
        if (at % 4) {
            tb.back().count += 1;
            at += 2;
        }
        std::shuffle(tb.begin(), tb.end(), rng);
        ddl_plan tp = nullptr;
        check(ddl_plan_create_typed(&tp, P, at, op, &topo, tb.data(), ntb, mode), "create_typed");
        std::vector<void *> raw(P);
        for (int r = 0; r < P; ++r)
            raw[r] = std::aligned_alloc(16, (at / 16 + 2) * 16);
        check(ddl_plan_execute(tp, raw.data(), nullptr, nullptr, nullptr), "typed execute");
        check(ddl_plan_destroy(tp), "typed destroy");
        for (int r = 0; r < P; ++r)
            std::free(raw[r]);
    }
    check(ddl_cache_clear(), "cache clear");
    if (g_live_allocs || g_live_streams || g_live_events)
        std::printf("FAILED: leaked %ld allocations, %ld streams, %ld events\n", g_live_allocs,
                    g_live_streams, g_live_events),
            std::exit(1);
    std::printf("ok %d cases, %ld launches checked\n", ncases, g_launches);
    return 0;
}
