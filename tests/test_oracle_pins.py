"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each test names what it pins.  None of them re-calls the oracle's own
formula: expected values come from closed forms, exact integer arithmetic,
hand-worked examples (derivation in the comments), invariants, or reductions
between schedules that must hold whatever the implementation.
"""
import itertools

import numpy as np
import pytest

import oracle as orc

def topologies(P):
    """Every schedule the oracle knows, at P ranks."""
    out = [("ring", dict(kind=orc.RING))]
    for k in (1, 2, 3):
        out.append((f"multiring{k}", dict(kind=orc.MULTIRING, k=k)))
    for r in range(1, P + 1):
        if P % r == 0:
            out.append((f"torus{r}x{P // r}", dict(kind=orc.TORUS2D, rows=r, cols=P // r)))
    return out


def run(bufs, **kw):
    bufs = [b.copy() for b in bufs]
    sent = orc.allreduce(bufs, **kw)
    return bufs, sent


# ---------------------------------------------------------------------------
# closed form: rank r holds r + 1 everywhere.  Every partial sum is an
# integer <= P(P+1)/2 <= 820 < 2^11, exact in binary32 and binary16, so any
# association order gives P(P+1)/2 (sum) or (P+1)/2 (mean) exactly.
# Pages: every worker ends with the same average (Baidu article, "总结";
# Sony article, the all-reduce paragraph).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 6, 8, 16, 40])
@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_closed_form_rank_plus_one(P, dtype):
    for L in sorted({0, 1, P - 1 if P > 1 else 1, P, 2 * P + 3, 37, 130}):
        for name, topo in topologies(P):
            for op, expect in ((orc.SUM, P * (P + 1) / 2), (orc.MEAN, (P + 1) / 2)):
                bufs = [np.full(L, r + 1, dtype=dtype) for r in range(P)]
                out, _ = run(bufs, op=op, **topo)
                for r in range(P):
                    assert np.array_equal(out[r], np.full(L, expect, dtype=dtype)), \
                        (name, P, L, op, r)


def test_closed_form_values_of_the_configs():
    # the values the five measured workloads' closed-form variants reach
    for P, s, m in ((4, 10, 2.5), (8, 36, 4.5), (16, 136, 8.5), (40, 820, 20.5)):
        bufs = [np.full(4 * P + 4, r + 1, dtype=np.float32) for r in range(P)]
        out, _ = run(bufs, op=orc.SUM)
        assert out[0][0] == s
        out, _ = run(bufs, op=orc.MEAN)
        assert out[P - 1][-1] == m


# ---------------------------------------------------------------------------
# exact integer sums: inputs are integers in [-64, 63]; every partial sum is
# an integer of magnitude <= 64 P < 2^11, so binary32 and binary16 adds are
# exact and the result is the integer sum whatever the order.  Checks that
# every rank's every element is counted exactly once.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_small_integer_sums_are_exact(dtype):
    rng = np.random.default_rng(11)
    for P in (2, 3, 4, 5, 7, 8, 12, 16):
        for L in (1, 5, P, 3 * P + 1, 61, 200):
            ints = rng.integers(-64, 64, size=(P, L))
            expect = ints.sum(axis=0)
            for name, topo in topologies(P):
                bufs = [ints[r].astype(dtype) for r in range(P)]
                out, _ = run(bufs, op=orc.SUM, **topo)
                for r in range(P):
                    assert np.array_equal(out[r].astype(np.int64), expect), (name, P, L, r)


# ---------------------------------------------------------------------------
# all ranks identical after the all-gather (pages: every worker ends with the
# same values), on random inputs where the order does change bits
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_all_ranks_identical(dtype):
    rng = np.random.default_rng(5)
    for P in (2, 3, 4, 6, 9, 16):
        for L in (1, P + 1, 97, 256):
            g = [rng.standard_normal(L).astype(dtype) for _ in range(P)]
            for name, topo in topologies(P):
                for op in (orc.SUM, orc.MEAN):
                    out, _ = run(g, op=op, **topo)
                    for r in range(1, P):
                        assert out[r].tobytes() == out[0].tobytes(), (name, P, L, op, r)


# ---------------------------------------------------------------------------
# association order: hand-worked examples.
#
# Ring of 3 ranks on 3 elements with q = 1, so chunk c is element c.
# Reduce-scatter step 0: position x sends chunk x to x+1, which adds it:
#   rank 1 elem 0 = g1 + g0, rank 2 elem 1 = g2 + g1, rank 0 elem 2 = g0 + g2.
# Step 1: position x sends chunk x-1:
#   rank 2 elem 0 = g2 + (g1 + g0)   -> ((g0 + g1) + g2)
#   rank 0 elem 1 = g0 + (g2 + g1)   -> ((g1 + g2) + g0)
#   rank 1 elem 2 = g1 + (g0 + g2)   -> ((g2 + g0) + g1)
# With g0 = 2^24, g1 = 1, g2 = -2^24 at every element:
#   elem 0: 2^24 + 1 is a tie between 2^24 and 2^24 + 2 -> even 2^24; minus
#           2^24 -> 0
#   elem 1: 1 - 2^24 = -16777215 (exact) + 2^24 -> 1
#   elem 2: 2^24 - 2^24 = 0, + 1 -> 1
# Starting each chain one rank later, or walking the ring the other way,
# gives a different vector, so the convention is pinned.
# ---------------------------------------------------------------------------
def test_ring3_chain_worked_example_f32():
    g = [np.full(3, v, dtype=np.float32) for v in (2.0 ** 24, 1.0, -2.0 ** 24)]
    out, _ = run(g, op=orc.SUM, q=1)
    for r in range(3):
        assert out[r].tolist() == [0.0, 1.0, 1.0]
    out, _ = run(g, op=orc.MEAN, q=1)
    third = float(np.float32(1.0) / np.float32(3.0))
    for r in range(3):
        assert out[r].tolist() == [0.0, third, third]


def test_ring3_chain_worked_example_f16():
    # same structure in binary16: 2048 + 1 ties to even 2048; 1 - 2048 = -2047
    g = [np.full(3, v, dtype=np.float16) for v in (2048.0, 1.0, -2048.0)]
    out, _ = run(g, op=orc.SUM, q=1)
    for r in range(3):
        assert out[r].astype(np.float64).tolist() == [0.0, 1.0, 1.0]


def test_ring_order_permutes_the_chain():
    # ring order (2, 0, 1): position x is rank order[x].  The chain of chunk
    # c starts at position c: elem 0 -> ((g2 + g0) + g1) = 1,
    # elem 1 -> ((g0 + g1) + g2) = 0, elem 2 -> ((g1 + g2) + g0) = 1.
    g = [np.full(3, v, dtype=np.float32) for v in (2.0 ** 24, 1.0, -2.0 ** 24)]
    out, _ = run(g, op=orc.SUM, q=1, ring_order=[2, 0, 1])
    for r in range(3):
        assert out[r].tolist() == [1.0, 0.0, 1.0]


def test_torus_2x2_worked_example():
    # 2x2 grid, rank (i, j) = 2i + j.  Row reduce-scatter makes the row sums
    # S_i = g(i,0) + g(i,1); the column all-reduce adds S_0 + S_1.  With
    # g(0,0) = 2^24, g(0,1) = 1, g(1,0) = 1, g(1,1) = -2^24:
    #   S_0 = 2^24 + 1 -> 2^24 (tie to even), S_1 = 1 - 2^24 (exact),
    #   y = 2^24 + (1 - 2^24) = 1 at every element.
    # A flat ring over ranks 0..3 would give element 0:
    #   ((2^24 + 1) + 1) + (-2^24) -> 0, so the two-level grouping is pinned.
    g = [np.full(4, v, dtype=np.float32) for v in (2.0 ** 24, 1.0, 1.0, -2.0 ** 24)]
    out, _ = run(g, op=orc.SUM, q=1, kind=orc.TORUS2D, rows=2, cols=2)
    for r in range(4):
        assert out[r].tolist() == [1.0] * 4
    ring, _ = run(g, op=orc.SUM, q=1)
    assert ring[0][0] == 0.0
    out, _ = run(g, op=orc.MEAN, q=1, kind=orc.TORUS2D, rows=2, cols=2)
    assert out[3].tolist() == [0.25] * 4


def test_torus_2x3_worked_example():
    # 2 rows x 3 columns, rank (i, j) = 3i + j; L = 6, q = 1.
    # Row split of 6 into 3: chunks {0,1}, {2,3}, {4,5}.  Row chunk c's chain
    # is (g(i,c) + g(i,c+1)) + g(i,c+2), columns mod 3.  Column j holds chunk
    # (j+1) mod 3 and splits it into 2 sub-chunks of one element: sub-chunk d
    # (d = 0 first element, d = 1 second) has chain S_d + S_{d+1}.
    # Put values only in row 0: g(0,0) = 2^24, g(0,1) = 1, g(0,2) = -2^24,
    # row 1 all zero.  Then S_1 = 0 and y = S_0 of the chunk:
    #   chunk 0 -> ((2^24 + 1) - 2^24) = 0, chunk 1 -> ((1 - 2^24) + 2^24) = 1,
    #   chunk 2 -> ((-2^24 + 2^24) + 1) = 1.
    vals = [2.0 ** 24, 1.0, -2.0 ** 24, 0.0, 0.0, 0.0]
    g = [np.full(6, v, dtype=np.float32) for v in vals]
    out, _ = run(g, op=orc.SUM, q=1, kind=orc.TORUS2D, rows=2, cols=3)
    for r in range(6):
        assert out[r].tolist() == [0.0, 0.0, 1.0, 1.0, 1.0, 1.0]


# ---------------------------------------------------------------------------
# association order on random data: the walk yields, for every element, the
# left-to-right chain the step rule implies (derived in the oracle's header:
# ring chunk c: g[o[c]], g[o[c+1]], ...; torus: row chains, then the column
# chain of row sums).  Brute force on tiny inputs.
# ---------------------------------------------------------------------------
def _chain_ring(g, order, c, dtype):
    P = len(order)
    acc = g[order[c % P]]
    for i in range(1, P):
        acc = dtype(acc + g[order[(c + i) % P]])
    return acc


def test_ring_chain_brute_force():
    rng = np.random.default_rng(7)
    for P in (2, 3, 4, 5, 8):
        for dtype in (np.float32, np.float16):
            L = 3 * P + 2
            q = 1
            g = [rng.uniform(-1, 1, L).astype(dtype) for _ in range(P)]
            order = list(rng.permutation(P))
            out, _ = run(g, op=orc.SUM, q=q, ring_order=order)
            b = orc.split(L, P, q)
            for c in range(P):
                for e in range(b[c], b[c + 1]):
                    want = _chain_ring([g[r][e] for r in range(P)], order, c, dtype)
                    assert out[0][e] == want, (P, dtype, c, e)


def test_torus_chain_brute_force():
    rng = np.random.default_rng(8)
    for R, C in ((2, 2), (2, 3), (3, 2), (3, 3), (4, 2)):
        for dtype in (np.float32, np.float16):
            P, L, q = R * C, 5 * R * C + 3, 1
            g = [rng.uniform(-1, 1, L).astype(dtype) for _ in range(P)]
            out, _ = run(g, op=orc.SUM, q=q, kind=orc.TORUS2D, rows=R, cols=C)
            cb = orc.split(L, C, q)
            for c in range(C):
                sub = orc.split(cb[c + 1] - cb[c], R, q)
                for d in range(R):
                    for e in range(cb[c] + sub[d], cb[c] + sub[d + 1]):
                        S = []
                        for i in range(R):
                            S.append(_chain_ring([g[i * C + j][e] for j in range(C)],
                                                 list(range(C)), c, dtype))
                        want = _chain_ring(S, list(range(R)), d, dtype)
                        assert out[0][e] == want, (R, C, c, d, e)


def test_order_matters_so_the_pins_bite():
    # at least 30% of elements change bits when the chain start moves by one
    # rank (P = 4, uniform inputs): a wrong convention cannot slip through
    rng = np.random.default_rng(9)
    P, L = 4, 4000
    g = [rng.uniform(-1, 1, L).astype(np.float32) for _ in range(P)]
    out, _ = run(g, op=orc.SUM, q=1)
    b = orc.split(L, P, 1)
    diff = 0
    for c in range(P):
        for e in range(b[c], b[c + 1]):
            shifted = _chain_ring([g[r][e] for r in range(P)], list(range(P)), c + 1,
                                  np.float32)
            diff += out[0][e] != shifted
    assert diff > 0.3 * L


# ---------------------------------------------------------------------------
# reductions between the schedules (special cases that must coincide)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_schedule_reductions(dtype):
    rng = np.random.default_rng(3)
    for P in (2, 3, 4, 6, 8):
        for L in (1, P - 1, 2 * P + 5, 203):
            g = [rng.standard_normal(L).astype(dtype) for _ in range(P)]
            for op in (orc.SUM, orc.MEAN):
                ring, _ = run(g, op=op)
                for topo in (dict(kind=orc.MULTIRING, k=1),
                             dict(kind=orc.TORUS2D, rows=1, cols=P),
                             dict(kind=orc.TORUS2D, rows=P, cols=1)):
                    other, _ = run(g, op=op, **topo)
                    assert all(a.tobytes() == b.tobytes() for a, b in zip(ring, other)), \
                        (P, L, op, topo)


def test_multiring_is_ring_over_its_parts():
    rng = np.random.default_rng(4)
    for P, k, L in ((4, 4, 203), (5, 3, 100), (16, 4, 1000)):
        g = [rng.standard_normal(L).astype(np.float32) for _ in range(P)]
        mr, _ = run(g, op=orc.MEAN, kind=orc.MULTIRING, k=k)
        parts = orc.split(L, k, 4)
        buckets = [(parts[j], parts[j + 1] - parts[j]) for j in range(k)]
        rb, _ = run(g, op=orc.MEAN, buckets=buckets)
        assert all(a.tobytes() == b.tobytes() for a, b in zip(mr, rb))


def test_two_ranks_is_one_add():
    rng = np.random.default_rng(1)
    for dtype in (np.float32, np.float16):
        g = [rng.standard_normal(101).astype(dtype) for _ in range(2)]
        out, _ = run(g, op=orc.SUM)
        assert np.array_equal(out[0], (g[0] + g[1]).astype(dtype))
        assert np.array_equal(out[1], (g[0] + g[1]).astype(dtype))


def test_one_rank_is_identity():
    rng = np.random.default_rng(2)
    for dtype in (np.float32, np.float16):
        g = [rng.standard_normal(50).astype(dtype)]
        for op in (orc.SUM, orc.MEAN):
            out, sent = run(g, op=op)
            assert out[0].tobytes() == g[0].tobytes()
            assert sent.tolist() == [0]


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_scaling_by_two_is_exact(dtype):
    # multiplying every input by 2 multiplies every rounded partial by 2
    # exactly, away from overflow and underflow
    rng = np.random.default_rng(6)
    for P in (3, 8, 16):
        g = [rng.uniform(0.25, 1, 300).astype(dtype) * rng.choice([-1, 1], 300).astype(dtype)
             for _ in range(P)]
        for name, topo in topologies(P):
            for op in (orc.SUM, orc.MEAN):
                a, _ = run(g, op=op, **topo)
                b, _ = run([(x * dtype(2)).astype(dtype) for x in g], op=op, **topo)
                assert np.array_equal(b[0], (a[0] * dtype(2)).astype(dtype)), (name, op)


def test_bucket_issue_order_does_not_matter():
    rng = np.random.default_rng(10)
    P, sizes = 6, [40, 8, 16, 104, 4, 24]
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).tolist()
    n = sum(sizes)
    g = [rng.standard_normal(n).astype(np.float32) for _ in range(P)]
    buckets = list(zip(offs, sizes))
    ref, _ = run(g, op=orc.MEAN, buckets=buckets)
    for perm in itertools.islice(itertools.permutations(range(len(sizes))), 0, 720, 97):
        out, _ = run(g, op=orc.MEAN, buckets=[buckets[i] for i in perm])
        assert all(a.tobytes() == b.tobytes() for a, b in zip(ref, out))


def test_each_bucket_is_its_own_allreduce():
    rng = np.random.default_rng(12)
    P, sizes = 4, [36, 20, 52]
    n = sum(sizes)
    g = [rng.standard_normal(n).astype(np.float32) for _ in range(P)]
    offs = [0, 36, 56]
    out, _ = run(g, op=orc.SUM, buckets=list(zip(offs, sizes)))
    for o, s in zip(offs, sizes):
        part, _ = run([x[o:o + s].copy() for x in g], op=orc.SUM)
        assert out[2][o:o + s].tobytes() == part[2].tobytes()


# ---------------------------------------------------------------------------
# the mean is a true division, not a reciprocal multiply
# ---------------------------------------------------------------------------
def test_mean_is_correctly_rounded_division():
    rng = np.random.default_rng(13)
    P, L = 40, 20000
    # put the whole sum on rank 0 so the final value is g0 / P exactly
    g = [rng.standard_normal(L).astype(np.float32)] + [np.zeros(L, np.float32)] * (P - 1)
    out, _ = run(g, op=orc.MEAN)
    assert np.array_equal(out[5], g[0] / np.float32(P))
    recip = g[0] * (np.float32(1) / np.float32(P))
    assert (recip != out[5]).mean() > 0.05


def test_mean_f16_division_correctly_rounded():
    x = np.arange(0, 0x7c00, dtype=np.uint16)  # all finite non-negative halfs
    # 14, 26, 28, 30, 56, 82 and 102 are rank counts where a binary32
    # reciprocal multiply, rounded to binary16, differs from the division
    for P in (2, 3, 5, 7, 10, 14, 16, 26, 28, 30, 40, 56, 82, 102):
        got = orc.f16_div(x, P)
        want = (x.view(np.float16).astype(np.float64) / P).astype(np.float16).view(np.uint16)
        assert np.array_equal(got, want), P


# ---------------------------------------------------------------------------
# traffic: a ring of m ranks over L elements moves 2 (m-1) L elements
# (Patarasuk & Yuan's bandwidth-optimal count, the Baidu article's reference
# 4); the torus moves the same in total.  Per rank: 2 (P-1)/P * N.
# ---------------------------------------------------------------------------
def test_traffic_identity():
    for P in (2, 3, 4, 5, 8, 16, 40):
        for L in (0, 1, P - 1, 7 * P, 1000, 4 * P * 25):
            for name, topo in topologies(P):
                sent = orc.traffic(P, L, **topo)
                assert int(sent.sum()) == 2 * (P - 1) * L, (name, P, L)
            if L % (P * 4) == 0:
                sent = orc.traffic(P, L)
                assert sent.tolist() == [2 * (P - 1) * L // P] * P


def test_traffic_of_the_pages_example():
    # Baidu article: a ~300M-parameter model has a 1.2 GB gradient and each
    # GPU must "send and receive about 2.4 GB"; 2.4 GB / 6 GB/s ~ 400 ms.
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden",
                           "baidu_traffic_example.json")) as f:
        ex = json.load(f)
    N, P = ex["params"], ex["gpus"]
    assert N * 4 == ex["gradient_bytes"]
    sent = orc.traffic(P, N)
    per_rank_bytes = int(sent[0]) * 4
    assert per_rank_bytes == 2 * (P - 1) * N // P * 4
    assert abs(per_rank_bytes - ex["per_gpu_bytes_each_way"]) / ex["per_gpu_bytes_each_way"] < 0.03
    assert abs(ex["per_gpu_bytes_each_way"] / ex["link_bytes_per_s"] - ex["est_seconds"]) < 0.001


# ---------------------------------------------------------------------------
# accuracy against the plain definition in binary64
# ---------------------------------------------------------------------------
def test_accuracy_against_f64():
    rng = np.random.default_rng(14)
    cases = [(40, np.float32, dict(kind=orc.RING), 1e-6, 1e-3),
             (16, np.float32, dict(kind=orc.MULTIRING, k=4), 1e-6, 1e-3),
             (16, np.float16, dict(kind=orc.TORUS2D, rows=4, cols=4), 2e-3, 1e-2)]
    for P, dtype, topo, tol, sigma in cases:
        L = 20000
        g = [(rng.standard_normal(L) * sigma).astype(np.float32).astype(dtype) for _ in range(P)]
        out, _ = run(g, op=orc.MEAN, **topo)
        ref = orc.sum_f64(g, op=orc.MEAN)
        err = np.linalg.norm(out[0].astype(np.float64) - ref) / np.linalg.norm(ref)
        assert err <= tol, (P, dtype, err)


def test_sum_f64_is_the_definition():
    g = [np.array([1.0, 2.0, -3.0], np.float32), np.array([0.5, 2.0, 3.0], np.float32)]
    assert orc.sum_f64(g).tolist() == [1.5, 4.0, 0.0]
    assert orc.sum_f64(g, op=orc.MEAN).tolist() == [0.75, 2.0, 0.0]


# ---------------------------------------------------------------------------
# the split rule
# ---------------------------------------------------------------------------
def test_split_rule():
    rng = np.random.default_rng(15)
    for _ in range(500):
        L = int(rng.integers(0, 5000))
        m = int(rng.integers(1, 50))
        q = int(rng.choice([1, 2, 4, 8]))
        b = orc.split(L, m, q)
        assert b[0] == 0 and b[m] == L
        assert all(b[i] <= b[i + 1] for i in range(m))
        assert all(b[i] % q == 0 for i in range(m) if b[i] < L)
        lens = [b[i + 1] - b[i] for i in range(m)]
        if L % q == 0:
            assert max(lens) - min(lens) <= q
        if q == 1:
            assert b == [c * L // m for c in range(m)] + [L]


def test_split_of_the_headline_bucket():
    # 4,687,500 fp32 elements over 40 ranks, quantum 4: chunks of 117,184 or
    # 117,188 elements, every one starting on a 16-byte boundary
    b = orc.split(4_687_500, 40, 4)
    lens = {b[i + 1] - b[i] for i in range(40)}
    assert lens == {117_184, 117_188}


def test_oracle_rejects_bad_arguments():
    g = [np.zeros(8, np.float32) for _ in range(4)]
    with pytest.raises(ValueError):
        orc.allreduce(g, kind=orc.TORUS2D, rows=3, cols=2)
    with pytest.raises(ValueError):
        orc.allreduce(g, ring_order=[0, 1, 1, 2])
    with pytest.raises(ValueError):
        orc.allreduce(g, buckets=[(0, 4), (2, 4)])
    with pytest.raises(ValueError):
        orc.allreduce(g, buckets=[(0, 4)])


# ---------------------------------------------------------------------------
# the SGD step after the all-reduce: w - lr * y, binary32, two roundings
# ---------------------------------------------------------------------------
def test_sgd_closed_forms():
    w = np.array([1.0, 0.5, -3.0, 0.0], np.float32)
    y = np.array([2.0, 1.0, -4.0, 0.0], np.float32)
    orc.sgd([w], y, 0.5)
    assert w.tolist() == [0.0, 0.0, -1.0, 0.0]
    # binary16 gradients are widened exactly
    w16 = np.array([1.0, 1.0], np.float32)
    orc.sgd([w16], np.array([2.0, -0.25], np.float16), 0.25)
    assert w16.tolist() == [0.5, 1.0625]


def test_sgd_two_roundings_not_fused():
    # lr * y rounds before the subtraction: pick values where a fused
    # multiply-add would round differently
    rng = np.random.default_rng(31)
    w = rng.standard_normal(100000).astype(np.float32)
    y = rng.standard_normal(100000).astype(np.float32)
    lr = np.float32(0.1)
    got = w.copy()
    orc.sgd([got], y, float(lr))
    want = w - (lr * y)                       # numpy float32: two roundings
    assert np.array_equal(got, want)
    fused = (w.astype(np.float64) - np.float64(lr) * y.astype(np.float64)).astype(np.float32)
    assert np.count_nonzero(fused != got) > 0


def test_sgd_every_replica_and_allreduce_then_update():
    # after a mean all-reduce every replica moves by the same step
    rng = np.random.default_rng(32)
    P, L = 5, 203
    g = [rng.standard_normal(L).astype(np.float32) for _ in range(P)]
    out, _ = run(g, op=orc.MEAN)
    ws = [np.full(L, 3.0, np.float32) for _ in range(P)]
    orc.sgd(ws, out[0], 0.01)
    for w in ws:
        assert np.array_equal(w, np.float32(3.0) - np.float32(0.01) * out[0])
