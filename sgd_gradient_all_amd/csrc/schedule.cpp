// schedule.cpp -- host schedule generator for the ring, multi-ring and
// 2D-torus all-reduce.
//
// The pages name the schedules but print none of their steps (the Baidu
// Ring-Allreduce article, part 4, names the ring in "总结" and cites
// Patarasuk & Yuan as its reference 4; "[论文解读] PowerAI DDL" names the
// multi-ring pattern in its ABSTRACT; the Sony "224秒训练ResNet-50" article
// gives the torus phases in "2D-Torus All-reduce" with Fig. 1 and a missing
// Fig. 2).  The readings taken:
//  - ring on m positions over pieces c = 0..m-1 of split(L, m, q):
//    reduce-scatter step t: position x sends piece (x-t) mod m to x+1, which
//    adds; all-gather step t: position x sends piece (x+1-t) mod m to x+1,
//    which copies.  After the reduce-scatter position (c-1) mod m owns piece c.
//  - multi-ring: bucket split into k parts, part j goes round ring j.
//  - torus: rank (i, j) = i*cols + j; row reduce-scatter; column j runs a
//    ring reduce-scatter + all-gather over row piece (j+1) mod cols (the one
//    it owns), split into rows sub-pieces; row all-gather.
//  - mean: the add that completes a piece's sum (last reduce-scatter step of
//    the last phase that reduces) also divides by P.
// Every piece of a segment starts on a multiple of q = 16 B / element size
// when the segment does, which keeps the kernels on dwordx4 accesses.
//
// The generator also lays out the kernels' tile tables: the tile prefix of
// every step's items and of the fused spans (tiles anchored at multiples of
// the tile size when the ranges average two tiles or more), the fused tile
// -> span table, and the broadcast's per-bucket tables.
#include "schedule.h"

#include <algorithm>

namespace ddl {

void split_segment(uint64_t L, int m, uint64_t q, std::vector<uint64_t> &b) {
    const uint64_t units = (L + q - 1) / q;
    b.assign((size_t)m + 1, 0);
    for (int c = 0; c < m; ++c)
        b[c] = std::min(L, q * (((uint64_t)c * units) / (uint64_t)m));
    b[m] = L;
}

namespace {

inline int wrap(int a, int m) { return ((a % m) + m) % m; }

class Builder {
  public:
    explicit Builder(Schedule &s) : s_(s) {}

    void emit(int step, int src, int dst, uint64_t off, uint64_t len, uint32_t flags) {
        if (len == 0)
            return;
        DevItem it;
        it.off = off;
        it.len = len;
        it.src = src;
        it.dst = dst;
        it.flags = flags | (off % s_.q == 0 ? kItemAligned : 0u);
        it.pad = 0;
        s_.items[step].push_back(it);
        s_.sent[src] += len;
        s_.step_bytes += (s_.step_kind[step] == DDL_K_REDUCE ? 3u : 2u) * len * (uint64_t)s_.esz;
    }

    // ring reduce-scatter of [off, off+L) over positions ring[0..m), steps
    // step0 .. step0+m-2.  In the last reducing phase (final) the last step
    // completes every chunk's sum: those items carry kItemFinal, and
    // kItemDivide for the mean.
    void reduce_scatter(const int *ring, int m, uint64_t off, uint64_t L, int step0,
                        bool final) {
        std::vector<uint64_t> b;
        split_segment(L, m, s_.q, b);
        const uint32_t last = final ? (kItemFinal | (s_.op == DDL_MEAN ? kItemDivide : 0u)) : 0u;
        for (int t = 0; t + 1 < m; ++t)
            for (int x = 0; x < m; ++x) {
                const int c = wrap(x - t, m);
                emit(step0 + t, ring[x], ring[(x + 1) % m], off + b[c], b[c + 1] - b[c],
                     t == m - 2 ? last : 0u);
            }
    }

    // ring all-gather of [off, off+L) over positions ring[0..m)
    void all_gather(const int *ring, int m, uint64_t off, uint64_t L, int step0) {
        std::vector<uint64_t> b;
        split_segment(L, m, s_.q, b);
        for (int t = 0; t + 1 < m; ++t)
            for (int x = 0; x < m; ++x) {
                const int c = wrap(x + 1 - t, m);
                emit(step0 + t, ring[x], ring[(x + 1) % m], off + b[c], b[c + 1] - b[c], 0u);
            }
    }

    void span(uint64_t off, uint64_t len, const std::vector<int> &chain) {
        if (len == 0)
            return;
        DevSpan sp;
        sp.off = off;
        sp.len = len;
        sp.chain_off = (uint32_t)s_.chains.size();
        sp.flags = off % s_.q == 0 ? kItemAligned : 0u;
        s_.spans.push_back(sp);
        for (int r : chain)
            s_.chains.push_back((uint8_t)r);
        s_.fused_bytes += 2ull * (uint64_t)s_.P * len * (uint64_t)s_.esz;
    }

    void ring_bucket(const Bucket &bk) {
        const int P = s_.P;
        std::vector<uint64_t> parts, b;
        split_segment(bk.len, s_.k, s_.q, parts);
        std::vector<int> chain(P);
        for (int j = 0; j < s_.k; ++j) {
            const int *ring = &s_.order[(size_t)j * P];
            const uint64_t off = bk.off + parts[j], len = parts[j + 1] - parts[j];
            reduce_scatter(ring, P, off, len, 0, true);
            all_gather(ring, P, off, len, P - 1);
            // piece c is summed starting at position c, round the ring
            split_segment(len, P, s_.q, b);
            for (int c = 0; c < P; ++c) {
                for (int i = 0; i < P; ++i)
                    chain[i] = ring[(c + i) % P];
                span(off + b[c], b[c + 1] - b[c], chain);
            }
        }
    }

    void torus_bucket(const Bucket &bk) {
        const int R = s_.rows, C = s_.cols, P = s_.P;
        std::vector<int> ring(std::max(R, C));
        std::vector<uint64_t> cb, sub;
        split_segment(bk.len, C, s_.q, cb);
        const int col_rs = C - 1, col_ag = C - 1 + R - 1, row_ag = C - 1 + 2 * (R - 1);
        for (int i = 0; i < R; ++i) {
            for (int j = 0; j < C; ++j)
                ring[j] = i * C + j;
            reduce_scatter(ring.data(), C, bk.off, bk.len, 0, R == 1);
        }
        for (int j = 0; j < C; ++j) {
            const int c = (j + 1) % C;
            for (int i = 0; i < R; ++i)
                ring[i] = i * C + j;
            reduce_scatter(ring.data(), R, bk.off + cb[c], cb[c + 1] - cb[c], col_rs, R > 1);
            all_gather(ring.data(), R, bk.off + cb[c], cb[c + 1] - cb[c], col_ag);
        }
        for (int i = 0; i < R; ++i) {
            for (int j = 0; j < C; ++j)
                ring[j] = i * C + j;
            all_gather(ring.data(), C, bk.off, bk.len, row_ag);
        }
        // sub-piece d of row piece c: row sums S_i = g(i,c) (+) g(i,c+1) ...,
        // then S_d (+) S_{d+1} (+) ... (rows and columns mod R, C)
        std::vector<int> chain(P);
        for (int c = 0; c < C; ++c) {
            split_segment(cb[c + 1] - cb[c], R, s_.q, sub);
            for (int d = 0; d < R; ++d) {
                for (int g = 0; g < R; ++g)
                    for (int h = 0; h < C; ++h)
                        chain[g * C + h] = ((d + g) % R) * C + (c + h) % C;
                span(bk.off + cb[c] + sub[d], sub[d + 1] - sub[d], chain);
            }
        }
    }

  private:
    Schedule &s_;
};

// Vectors per lane of the step kernels, from the mean item length.  Measured
// on MI355X: long items (a 300M-element bucket over 8 ranks, 37.5M-element
// chunks) run best with one vector per lane -- fewer requests in flight per
// wave; chunks of ~10^5 elements with two; short items (the ResNet-50
// tensors, ~2.5K-element chunks) with four, which keeps the number of
// workgroups -- each of which looks its item up -- low.
int pick_step_vpl(const Schedule &s) {
    uint64_t total = 0, count = 0;
    for (const auto &step : s.items)
        for (const DevItem &it : step) {
            total += it.len;
            ++count;
        }
    const uint64_t mean = count ? total / count : 0;
    if (mean >= (4ull << 20))
        return 1;
    if (mean >= (64ull << 10))
        return 2;
    return 4;
}

// Whether a table's tiles are anchored at multiples of the tile size: when
// its ranges average at least 2 tiles.  Measured on MI355X (paired, fused
// tables): +3..+7% for the one-kernel pass at 40 and 16 ranks, +1..+2% for
// the two-kernel pass, including the ResNet-50 multi-ring table whose spans
// average 2.4 tiles; the ResNet-50 step items (0.6 tiles) stay unanchored.
bool pick_anchor(const std::vector<std::pair<uint64_t, uint64_t>> &ranges, uint64_t tile) {
    const int forced = tuning(DDL_TUNE_ANCHOR);
    if (forced == 1 || forced == 2)
        return forced == 2;
    uint64_t total = 0;
    for (const auto &r : ranges)
        total += r.second;
    return !ranges.empty() && total / ranges.size() >= 2 * tile;
}

// Tile prefix of a list of ranges (offset, length).
bool tiles_prefix(const std::vector<std::pair<uint64_t, uint64_t>> &ranges, uint64_t tile,
                  bool anchor, std::vector<uint32_t> &pre) {
    pre.assign(ranges.size() + 1, 0);
    uint64_t acc = 0;
    for (size_t i = 0; i < ranges.size(); ++i) {
        acc += tile_count(ranges[i].second, tile_shift(ranges[i].first, tile, anchor), tile);
        if (acc > 0x7fffffffull)
            return false;
        pre[i + 1] = (uint32_t)acc;
    }
    return true;
}

}  // namespace

int build_schedule(Schedule &s, int P, uint64_t n, int dtype, int op, const ddl_topo &topo,
                   const ddl_bucket *buckets, int nbuckets, bool exact) {
    if (P < 1 || P > DDL_MAX_RANKS)
        return DDL_E_ARG;
    if (dtype != DDL_F32 && dtype != DDL_F16)
        return DDL_E_ARG;
    if (op != DDL_SUM && op != DDL_MEAN)
        return DDL_E_ARG;
    s = Schedule();
    s.P = P;
    s.n = n;
    s.dtype = dtype;
    s.esz = dtype == DDL_F32 ? 4 : 2;
    s.q = (uint64_t)(kVecBytes / s.esz);
    s.op = op;
    s.kind = topo.kind;
    switch (topo.kind) {
    case DDL_RING:
        s.k = 1;
        break;
    case DDL_MULTIRING:
        if (topo.k < 1 || topo.k > 1024)
            return DDL_E_ARG;
        s.k = topo.k;
        break;
    case DDL_TORUS2D:
        if (topo.rows < 1 || topo.cols < 1 || topo.rows * topo.cols != P || topo.ring_order)
            return DDL_E_ARG;
        s.rows = topo.rows;
        s.cols = topo.cols;
        break;
    default:
        return DDL_E_ARG;
    }
    if (topo.kind != DDL_TORUS2D) {
        s.order.resize((size_t)s.k * P);
        for (int j = 0; j < s.k; ++j) {
            std::vector<char> seen(P, 0);
            for (int x = 0; x < P; ++x) {
                const int r = topo.ring_order ? topo.ring_order[(size_t)j * P + x] : x;
                if (r < 0 || r >= P || seen[r])
                    return DDL_E_ARG;
                seen[r] = 1;
                s.order[(size_t)j * P + x] = r;
            }
        }
    }

    // buckets: NULL with nbuckets == 0 means one bucket over [0, n)
    if (nbuckets < 0 || (nbuckets > 0 && !buckets))
        return DDL_E_NULL;
    if (nbuckets == 0) {
        if (n > 0)
            s.buckets.push_back({0, n});
    } else {
        std::vector<Bucket> sorted;
        for (int b = 0; b < nbuckets; ++b) {
            const uint64_t off = buckets[b].offset, len = buckets[b].count;
            if (off > n || len > n - off)
                return DDL_E_BUCKETS;
            s.buckets.push_back({off, len});
            if (len)
                sorted.push_back({off, len});
        }
        std::sort(sorted.begin(), sorted.end(),
                  [](const Bucket &a, const Bucket &b) { return a.off < b.off; });
        uint64_t at = 0;
        for (const Bucket &bk : sorted) {
            if (exact ? bk.off != at : bk.off < at)
                return DDL_E_BUCKETS;
            at = bk.off + bk.len;
        }
        if (exact && at != n)
            return DDL_E_BUCKETS;
    }
    const int nb = (int)s.buckets.size();

    if (s.kind == DDL_TORUS2D) {
        s.nsteps = 2 * (s.cols - 1) + 2 * (s.rows - 1);
        s.step_kind.assign(s.nsteps, DDL_K_GATHER);
        for (int t = 0; t < s.cols - 1 + s.rows - 1; ++t)
            s.step_kind[t] = DDL_K_REDUCE;
        s.group = s.cols == 1 ? P : s.cols;
    } else {
        s.nsteps = 2 * (P - 1);
        s.step_kind.assign(s.nsteps, DDL_K_GATHER);
        for (int t = 0; t < P - 1; ++t)
            s.step_kind[t] = DDL_K_REDUCE;
        s.group = P;
    }
    s.items.assign(s.nsteps, {});
    s.item_at.assign(s.nsteps, std::vector<uint32_t>(nb + 1, 0));
    s.span_at.assign(nb + 1, 0);
    s.sent.assign(P, 0);

    Builder bld(s);
    for (int b = 0; b < nb; ++b) {
        for (int st = 0; st < s.nsteps; ++st)
            s.item_at[st][b] = (uint32_t)s.items[st].size();
        s.span_at[b] = (uint32_t)s.spans.size();
        if (s.kind == DDL_TORUS2D)
            bld.torus_bucket(s.buckets[b]);
        else
            bld.ring_bucket(s.buckets[b]);
    }
    for (int st = 0; st < s.nsteps; ++st)
        s.item_at[st][nb] = (uint32_t)s.items[st].size();
    s.span_at[nb] = (uint32_t)s.spans.size();

    s.prefix.assign(s.nsteps, {});
    s.step_vpl = pick_step_vpl(s);
    std::vector<std::pair<uint64_t, uint64_t>> ranges;
    const uint64_t stile = step_tile_elems(s.esz, s.step_vpl);
    for (int st = 0; st < s.nsteps; ++st)
        for (const DevItem &it : s.items[st])
            ranges.emplace_back(it.off, it.len);
    s.step_anchor = pick_anchor(ranges, stile);
    for (int st = 0; st < s.nsteps; ++st) {
        ranges.clear();
        for (const DevItem &it : s.items[st])
            ranges.emplace_back(it.off, it.len);
        if (!tiles_prefix(ranges, stile, s.step_anchor, s.prefix[st]))
            return DDL_E_ARG;
    }
    ranges.clear();
    for (const DevSpan &sp : s.spans)
        ranges.emplace_back(sp.off, sp.len);
    s.fused_anchor = pick_anchor(ranges, fused_tile_elems(s.esz));
    if (!tiles_prefix(ranges, fused_tile_elems(s.esz), s.fused_anchor, s.span_prefix))
        return DDL_E_ARG;
    // one load instead of a search per workgroup: the fused kernels' tiles
    // are short-lived, so the lookup's latency is a measurable share of them
    s.span_of_tile.resize(s.span_prefix.back());
    for (size_t i = 0; i < s.spans.size(); ++i)
        for (uint32_t t = s.span_prefix[i]; t < s.span_prefix[i + 1]; ++t)
            s.span_of_tile[t] = (uint32_t)i;
    s.tiny_prefix.assign(s.spans.size() + 1, 0);
    for (size_t i = 0; i < s.spans.size(); ++i) {
        const bool tiny = s.spans[i].len <= kTinySpanMax;
        if (tiny)
            s.tiny.push_back((uint32_t)i);
        s.tiny_prefix[i + 1] = s.tiny_prefix[i] + (tiny ? 1u : 0u);
    }
    ranges.clear();
    for (const Bucket &b : s.buckets) {
        s.bk_spans.push_back({b.off, b.len, 0u, b.off % s.q == 0 ? (uint32_t)kItemAligned : 0u});
        ranges.emplace_back(b.off, b.len);
    }
    if (!tiles_prefix(ranges, fused_tile_elems(s.esz), true, s.bk_prefix))
        return DDL_E_ARG;
    s.bk_of_tile.resize(s.bk_prefix.back());
    for (size_t i = 0; i < s.buckets.size(); ++i)
        for (uint32_t t = s.bk_prefix[i]; t < s.bk_prefix[i + 1]; ++t)
            s.bk_of_tile[t] = (uint32_t)i;
    if (!check_schedule(s))
        return DDL_E_ARG;  // cannot happen for the schedules above
    return DDL_OK;
}

bool check_schedule(const Schedule &s) {
    struct Iv {
        uint64_t lo, hi;
        bool write;
    };
    std::vector<std::vector<Iv>> per_rank(s.P);
    for (int st = 0; st < s.nsteps; ++st) {
        for (auto &v : per_rank)
            v.clear();
        for (const DevItem &it : s.items[st]) {
            if (it.src == it.dst)
                return false;
            per_rank[it.dst].push_back({it.off, it.off + it.len, true});
            per_rank[it.src].push_back({it.off, it.off + it.len, false});
        }
        // an item touches each rank at most once, so any overlap on a rank
        // is between two items; it is a race unless both only read
        for (auto &v : per_rank) {
            std::sort(v.begin(), v.end(), [](const Iv &a, const Iv &b) { return a.lo < b.lo; });
            uint64_t end = 0;
            bool has_write = false;
            for (const Iv &iv : v) {
                if (iv.lo < end) {
                    if (iv.write || has_write)
                        return false;
                    end = std::max(end, iv.hi);
                } else {
                    end = iv.hi;
                    has_write = false;
                }
                has_write = has_write || iv.write;
            }
        }
    }
    return true;
}

}  // namespace ddl
