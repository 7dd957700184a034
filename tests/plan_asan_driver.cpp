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
