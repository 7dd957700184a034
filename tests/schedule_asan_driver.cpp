// schedule_asan_driver.cpp -- host-only driver of the schedule generator,
// built by the test suite with AddressSanitizer and UndefinedBehaviorSanitizer
// (g++, no GPU code).  For random rank counts, lengths, topologies, ring
// orders and bucket lists it checks, independently of the oracle:
//  - every element of every rank is written exactly once by the reduce
//    phase's final adds and the all-gather copies together (it ends up
//    holding the reduced value), and each chunk's final add happens once;
//  - within a step no element is written by one pair and touched by another
//    (the generator's own race check must agree);
//  - the traffic identity: the ranks send 2 (P-1) L elements per ring segment;
//  - every fused span's chain is a permutation of the ranks, and the spans of
//    a bucket tile it exactly;
//  - the fused tile -> span table agrees with the spans' tile prefix.
// Exit status 0 when all checks pass; prints the failing case otherwise.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../sgd_gradient_all_amd/csrc/schedule.h"

using namespace ddl;

// The library's tuning knobs live with the plans (plan.cpp, not linked
// here).  The generator reads one, tile anchoring, which this driver cycles
// through automatic / never / always.
static int g_anchor = 0;
namespace ddl {
int tuning(int knob) { return knob == DDL_TUNE_ANCHOR ? g_anchor : 0; }
}  // namespace ddl

static int fail(const char *what, int P, uint64_t n, int kind) {
    std::printf("FAIL %s: P=%d n=%llu kind=%d\n", what, P, (unsigned long long)n, kind);
    return 1;
}

int main(int argc, char **argv) {
    const int cases = argc > 1 ? std::atoi(argv[1]) : 400;
    std::mt19937_64 rng(12345);
    for (int cs = 0; cs < cases; ++cs) {
        g_anchor = cs % 3;
        const int P = 1 + (int)(rng() % 24);
        const uint64_t n = rng() % 3000;
        const int dtype = (int)(rng() % 2);
        const int op = (int)(rng() % 2);
        ddl_topo topo{};
        topo.kind = (int)(rng() % 3);
        std::vector<int> order;
        if (topo.kind == DDL_TORUS2D) {
            std::vector<int> divs;
            for (int d = 1; d <= P; ++d)
                if (P % d == 0)
                    divs.push_back(d);
            topo.rows = divs[rng() % divs.size()];
            topo.cols = P / topo.rows;
        } else {
            topo.k = topo.kind == DDL_MULTIRING ? 1 + (int)(rng() % 4) : 1;
            const int rings = topo.kind == DDL_MULTIRING ? topo.k : 1;
            for (int j = 0; j < rings; ++j) {
                std::vector<int> perm(P);
                for (int x = 0; x < P; ++x)
                    perm[x] = x;
                std::shuffle(perm.begin(), perm.end(), rng);
                order.insert(order.end(), perm.begin(), perm.end());
            }
            if (rng() % 2)
                topo.ring_order = order.data();
        }
        // a random bucket list tiling [0, n), in reverse order
        std::vector<ddl_bucket> buckets;
        uint64_t at = 0;
        while (at < n) {
            const uint64_t len = std::min<uint64_t>(n - at, 1 + rng() % 700);
            buckets.push_back({(size_t)at, (size_t)len, nullptr});
            at += len;
        }
        std::reverse(buckets.begin(), buckets.end());

        Schedule s;
        const int rc = build_schedule(s, P, n, dtype, op, topo, buckets.data(),
                                      (int)buckets.size());
        if (rc != DDL_OK)
            return fail("build_schedule", P, n, topo.kind);
        if (!check_schedule(s))
            return fail("check_schedule", P, n, topo.kind);

        // final adds + gather deliveries: exactly once per element per rank
        std::vector<std::vector<int>> got(P, std::vector<int>(n, 0));
        std::vector<int> finals(n, 0);
        for (int st = 0; st < s.nsteps; ++st)
            for (const DevItem &it : s.items[st]) {
                const bool reduce = s.step_kind[st] == DDL_K_REDUCE;
                if (reduce && !(it.flags & kItemFinal))
                    continue;
                for (uint64_t e = it.off; e < it.off + it.len; ++e) {
                    got[it.dst][e] += 1;
                    if (reduce)
                        finals[e] += 1;
                }
            }
        for (uint64_t e = 0; e < n; ++e) {
            if (P > 1 && finals[e] != 1)
                return fail("one final add per element", P, n, topo.kind);
            for (int r = 0; r < P && P > 1; ++r)
                if (got[r][e] != 1)
                    return fail("every rank receives the reduced value once", P, n, topo.kind);
        }
        // traffic: 2 (P-1) L per ring segment, so 2 (P-1) n in total
        uint64_t sent = 0;
        for (uint64_t v : s.sent)
            sent += v;
        if (sent != 2ull * (uint64_t)(P - 1) * n)
            return fail("traffic identity", P, n, topo.kind);
        // fused spans tile every bucket; chains are permutations
        for (size_t b = 0; b < s.buckets.size(); ++b) {
            uint64_t covered = 0;
            for (uint32_t i = s.span_at[b]; i < s.span_at[b + 1]; ++i) {
                const DevSpan &sp = s.spans[i];
                if (sp.off < s.buckets[b].off || sp.off + sp.len > s.buckets[b].off + s.buckets[b].len)
                    return fail("span inside its bucket", P, n, topo.kind);
                covered += sp.len;
                std::vector<int> seen(P, 0);
                for (int r = 0; r < P; ++r) {
                    const int c = s.chains[sp.chain_off + r];
                    if (c < 0 || c >= P || seen[c]++)
                        return fail("chain is a permutation", P, n, topo.kind);
                }
            }
            if (covered != s.buckets[b].len)
                return fail("spans tile the bucket", P, n, topo.kind);
        }
        if (s.bk_of_tile.size() != s.bk_prefix.back() || s.bk_spans.size() != s.buckets.size())
            return fail("broadcast bucket tables", P, n, topo.kind);
        for (size_t t = 0; t < s.bk_of_tile.size(); ++t) {
            const uint32_t i = s.bk_of_tile[t];
            if (i >= s.buckets.size() || s.bk_prefix[i] > t || t >= s.bk_prefix[i + 1])
                return fail("tile -> bucket table", P, n, topo.kind);
        }
        if (s.span_of_tile.size() != s.span_prefix.back())
            return fail("one table entry per fused tile", P, n, topo.kind);
        for (size_t t = 0; t < s.span_of_tile.size(); ++t) {
            const uint32_t i = s.span_of_tile[t];
            if (i >= s.spans.size() || s.span_prefix[i] > t || t >= s.span_prefix[i + 1])
                return fail("tile -> span table", P, n, topo.kind);
        }
    }
    std::printf("ok %d cases\n", cases);
    return 0;
}
