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

#include "fake_device.inc"

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

static void expect(int rc, int want, const char *what) {
    if (rc != want) {
        std::printf("FAILED: %s returned %d, expected %d\n", what, rc, want);
        std::exit(1);
    }
}

// A destroyed handle, a second destroy, and a pointer that was never a
// plan are argument errors: the handle is looked up in the library's
// registry of live plans before anything is touched.
static void stale_handles() {
    ddl_topo ring = {DDL_RING, 1, 0, 0, nullptr};
    const size_t n = 4096;
    std::vector<void *> bufs(4);
    for (auto &b : bufs)
        b = std::aligned_alloc(16, n * 4);
    hipStream_t s;
    (void)hipStreamCreateWithFlags(&s, 0);
    ddl_plan plan = nullptr;
    check(ddl_plan_create(&plan, 4, n, DDL_F32, DDL_SUM, &ring, nullptr, 0, DDL_FUSED), "create");
    std::vector<void *> w0(bufs);
    expect(ddl_plan_execute_lars_noalloc(plan, bufs.data(), w0.data(), 1, 0.1f, 0.01, 1e-6,
                                         nullptr, nullptr, s, nullptr),
           DDL_E_UNBOUND, "allocation-free LARS before the plan has run");
    check(ddl_plan_execute(plan, bufs.data(), nullptr, s, nullptr), "execute");
    // the allocation-free call makes no device allocation
    const long allocs = g_live_allocs;
    check(ddl_plan_execute_lars_noalloc(plan, bufs.data(), w0.data(), 1, 0.1f, 0.01, 1e-6,
                                        nullptr, nullptr, s, nullptr),
          "allocation-free LARS");
    if (g_live_allocs != allocs)
        fail("the allocation-free LARS call allocated device memory");
    check(ddl_plan_destroy(plan), "destroy");
    expect(ddl_plan_destroy(plan), DDL_E_ARG, "second destroy");
    expect(ddl_plan_execute(plan, bufs.data(), nullptr, s, nullptr), DDL_E_ARG,
           "execute after destroy");
    std::vector<void *> w(bufs);
    expect(ddl_plan_execute_sgd(plan, bufs.data(), w.data(), 4, 0.1f, 1, nullptr, s, nullptr),
           DDL_E_ARG, "SGD after destroy");
    expect(ddl_plan_execute_lars(plan, bufs.data(), w.data(), 4, 0.1f, 0.01, 1e-6, nullptr,
                                 nullptr, s, nullptr),
           DDL_E_ARG, "LARS after destroy");
    size_t hbm = 0;
    expect(ddl_plan_traffic(plan, nullptr, &hbm), DDL_E_ARG, "traffic after destroy");
    expect(ddl_plan_set_coalesce_bytes(plan, 1), DDL_E_ARG, "coalesce after destroy");
    expect(ddl_plan_set_profiling(plan, 1), DDL_E_ARG, "profiling after destroy");
    int v = 0;
    expect(ddl_plan_num_steps(plan, &v), DDL_E_ARG, "num_steps after destroy");
    // an address that never was a plan
    int junk[64] = {};
    ddl_plan fake = reinterpret_cast<ddl_plan>(junk);
    expect(ddl_plan_destroy(fake), DDL_E_ARG, "destroy of a foreign pointer");
    expect(ddl_plan_execute(fake, bufs.data(), nullptr, s, nullptr), DDL_E_ARG,
           "execute of a foreign pointer");
    expect(ddl_plan_destroy(nullptr), DDL_E_NULL, "destroy of NULL");
    (void)hipStreamDestroy(s);
    for (auto &b : bufs)
        std::free(b);
}

// The one-shot cache makes room by destroying idle plans, but never one
// whose execution was captured into a HIP graph: the graph's replays read
// its tables.  ddl_cache_clear keeps those too.
// ddl_plan_event_groups reports the groups that a call with one ready event
// per bucket forms: one event per reported group, passed for each of its
// buckets, gives the same launches with one wait per group.
static void event_groups_match() {
    std::mt19937_64 rng(777);
    auto uni = [&](int lo, int hi) { return lo + (int)(rng() % (uint64_t)(hi - lo + 1)); };
    const size_t thresholds[] = {0, 1, 4096, 65536, 1 << 20, (size_t)1 << 30};
    for (int c = 0; c < 48; ++c) {
        const int P = uni(2, 9), nb = uni(1, 24);
        std::vector<ddl_bucket> bk(nb);
        size_t n = 0;
        for (int b = 0; b < nb; ++b) {
            const size_t cnt = uni(0, 4) == 0 ? (size_t)uni(1, 40) : (size_t)uni(40, 50000);
            bk[b] = {n, cnt, nullptr};
            n += cnt;
        }
        std::shuffle(bk.begin(), bk.end(), rng);
        ddl_topo topo = {DDL_RING, 1, 0, 0, nullptr};
        const ddl_mode mode = c % 2 ? DDL_STEPWISE : DDL_FUSED;
        ddl_plan plan = nullptr;
        check(ddl_plan_create(&plan, P, n, DDL_F32, DDL_SUM, &topo, bk.data(), nb, mode),
              "create");
        const bool ordered = uni(0, 1);
        check(ddl_plan_set_coalesce_bytes(plan, thresholds[c % 6]), "coalesce");
        check(ddl_plan_set_ordered_events(plan, ordered), "ordered");
        const int G = ddl_plan_event_groups(plan, nullptr, 0);
        if (G < 1 || G > nb)
            fail("event_groups count");
        std::vector<int> last(G + 1, -5);
        if (ddl_plan_event_groups(plan, last.data(), G) != G || last[G] != -5 ||
            last[G - 1] != nb - 1)
            fail("event_groups list");
        for (int g = 1; g < G; ++g)
            if (last[g] <= last[g - 1])
                fail("event_groups not increasing");
        if (thresholds[c % 6] == 0 && G != nb)
            fail("event_groups without a threshold");
        int first = -5;
        if (ddl_plan_event_groups(plan, &first, 1) != G || first != last[0])
            fail("event_groups with a short array");
        if (ddl_plan_event_groups(plan, nullptr, 1) != DDL_E_ARG ||
            ddl_plan_event_groups(plan, last.data(), -1) != DDL_E_ARG ||
            ddl_plan_event_groups(nullptr, nullptr, 0) != DDL_E_NULL)
            fail("event_groups argument checks");
        std::vector<void *> bufs(P);
        for (int r = 0; r < P; ++r)
            bufs[r] = std::aligned_alloc(16, ((n * 4 + 15) / 16 + 1) * 16);
        std::vector<hipEvent_t> ev(nb), gev(G);
        std::vector<void *> own(nb), shared(nb);
        for (int b = 0; b < nb; ++b) {
            (void)hipEventCreate(&ev[b]);
            own[b] = ev[b];
            g_caller_events.insert(ev[b]);
        }
        for (int g = 0, b = 0; g < G; ++g) {
            (void)hipEventCreate(&gev[g]);
            g_caller_events.insert(gev[g]);
            for (; b <= last[g]; ++b)
                shared[b] = gev[g];
        }
        hipStream_t s;
        (void)hipStreamCreateWithFlags(&s, 0);
        g_caller_waits = 0;
        long l0 = g_launches;
        check(ddl_plan_execute(plan, bufs.data(), own.data(), s, nullptr), "execute own");
        const long w_own = g_caller_waits, l_own = g_launches - l0;
        g_caller_waits = 0;
        l0 = g_launches;
        check(ddl_plan_execute(plan, bufs.data(), shared.data(), s, nullptr), "execute shared");
        const long w_shared = g_caller_waits, l_shared = g_launches - l0;
        if (l_own != l_shared)
            fail("group events change the launches");
        if (w_shared != G || w_own != (ordered ? G : nb))
            fail("waits on the caller's events");
        check(ddl_plan_destroy(plan), "destroy");
        for (int b = 0; b < nb; ++b)
            (void)hipEventDestroy(ev[b]);
        for (int g = 0; g < G; ++g)
            (void)hipEventDestroy(gev[g]);
        g_caller_events.clear();
        (void)hipStreamDestroy(s);
        for (int r = 0; r < P; ++r)
            std::free(bufs[r]);
    }
}

static void captured_plans_stay_cached() {
    ddl_topo ring = {DDL_RING, 1, 0, 0, nullptr};
    const size_t n = 10000;
    std::vector<void *> bufs(8);
    for (auto &b : bufs)
        b = std::aligned_alloc(16, (n + 64) * 4);
    hipStream_t s;
    (void)hipStreamCreateWithFlags(&s, 0);
    // a stream under capture (fake: its token holds kCapturingStream)
    hipStream_t cap = reinterpret_cast<hipStream_t>(new int(kCapturingStream));
    for (int mode = 0; mode < 2; ++mode) {
        ddl_bucket all = {0, n, nullptr};
        check(ddl_allreduce(bufs.data(), 8, n, DDL_F32, DDL_MEAN, &ring, &all, 1, (ddl_mode)mode,
                            s, nullptr),
              "eager call before the capture");
        check(ddl_allreduce(bufs.data(), 8, n, DDL_F32, DDL_MEAN, &ring, &all, 1, (ddl_mode)mode,
                            cap, nullptr),
              "captured call");
    }
    if (g_captured_tables.empty())
        fail("no launch was enqueued on the capturing stream");
    // 150 other shapes push the cache past its bound many times over
    for (int i = 0; i < 150; ++i) {
        ddl_bucket all = {0, n - 1 - (size_t)i, nullptr};
        check(ddl_allreduce(bufs.data(), 8, all.count, DDL_F32, DDL_SUM, &ring, &all, 1,
                            DDL_FUSED, s, nullptr),
              "one-shot call");
    }
    size_t cached = 0;
    check(ddl_cache_count(&cached), "cache count");
    if (cached > 64)
        fail("cache above its bound");
    for (const void *t : g_captured_tables)
        if (!live_address(t))
            fail("a captured plan's tables were freed by the cache");
    check(ddl_cache_clear(), "cache clear with captured plans");
    check(ddl_cache_count(&cached), "cache count");
    if (cached != 2)
        fail("ddl_cache_clear dropped a captured plan, or kept another one");
    for (const void *t : g_captured_tables)
        if (!live_address(t))
            fail("ddl_cache_clear freed a captured plan's tables");
    delete reinterpret_cast<int *>(cap);
    (void)hipStreamDestroy(s);
    for (auto &b : bufs)
        std::free(b);
}

// The allocation-free call on more new streams than the plan has spare
// tracking events for: once they are used up it reports DDL_E_NOMEM before
// enqueuing anything, so that no work it cannot track is left in flight.
static void noalloc_out_of_tracking_events() {
    ddl_topo ring = {DDL_RING, 1, 0, 0, nullptr};
    const int P = 4;
    const size_t n = 8192;
    std::vector<void *> bufs(P), w(P);
    for (int r = 0; r < P; ++r) {
        bufs[r] = std::aligned_alloc(16, n * 4);
        w[r] = std::aligned_alloc(16, n * 4);
    }
    hipStream_t s0;
    (void)hipStreamCreateWithFlags(&s0, 0);
    ddl_plan plan = nullptr;
    check(ddl_plan_create(&plan, P, n, DDL_F32, DDL_SUM, &ring, nullptr, 0, DDL_FUSED), "create");
    check(ddl_plan_execute(plan, bufs.data(), nullptr, s0, nullptr), "binding call");
    std::vector<hipStream_t> streams;
    int rc = DDL_OK;
    for (int i = 0; i < 64 && rc == DDL_OK; ++i) {
        hipStream_t si;
        (void)hipStreamCreateWithFlags(&si, 0);
        streams.push_back(si);
        const long k0 = g_launches;
        rc = ddl_plan_execute_lars_noalloc(plan, bufs.data(), w.data(), P, 0.1f, 0.01, 1e-6,
                                           nullptr, nullptr, si, nullptr);
        if (rc != DDL_OK && g_launches != k0)
            fail("an allocation-free call without a tracking event launched kernels");
    }
    expect(rc, DDL_E_NOMEM, "allocation-free call once the spare tracking events are used");
    check(ddl_plan_destroy(plan), "destroy");
    for (hipStream_t si : streams)
        (void)hipStreamDestroy(si);
    (void)hipStreamDestroy(s0);
    for (int r = 0; r < P; ++r) {
        std::free(bufs[r]);
        std::free(w[r]);
    }
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
        check(ddl_plan_set_ordered_events(plan, uni(0, 1)), "ordered events");
        check(ddl_plan_set_coalesce_bytes(plan, uni(0, 1) ? 0 : (size_t)uni(1, 1 << 22)),
              "coalesce");
        if (mode == DDL_FUSED)
            check(ddl_plan_set_fused_passes(plan, uni(0, 2)), "passes");
        else
            check(ddl_plan_set_step_form(plan, uni(0, 2)), "step form");
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
            check(ddl_plan_execute_lars_noalloc(plan, bufs.data(), w.data(), uni(0, 1) ? 1 : P,
                                                0.01f, 0.01, 1e-6, nullptr,
                                                uni(0, 1) ? evp.data() : nullptr, s, nullptr),
                  "execute_lars_noalloc");
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
    stale_handles();
    noalloc_out_of_tracking_events();
    event_groups_match();
    if (g_live_allocs || g_live_streams || g_live_events)
        std::printf("FAILED: leaked %ld allocations, %ld streams, %ld events\n", g_live_allocs,
                    g_live_streams, g_live_events),
            std::exit(1);
    captured_plans_stay_cached();
    std::printf("ok %d cases, %ld launches checked\n", ncases, g_launches);
    return 0;
}
