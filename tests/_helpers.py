"""Shared helpers of the test suite: workload plumbing, host/device inputs,
and oracle expectations (full or at sampled elements)."""
import sys

import numpy as np

import oracle as orc
import synth

KINDS = {"ring": orc.RING, "multiring": orc.MULTIRING, "torus2d": orc.TORUS2D}
OPS = {"sum": orc.SUM, "mean": orc.MEAN}


def np_dtype(dt):
    return np.float32 if dt == "f32" else np.float16


def synth_dtype(dt):
    return synth.F32 if dt == "f32" else synth.F16


def say(*a):
    """Name the case on stdout before a GPU step (flushed)."""
    print(*a, flush=True)
    sys.stdout.flush()


def ddl_topo(w):
    import sgd_gradient_all_amd as ddl
    return ddl.topo(w.topo, w.k, w.rows, w.cols)


def host_inputs(w, first=0, count=None, dist=None):
    count = w.n - first if count is None else count
    return [synth.fill_host(count, synth_dtype(w.dtype), dist or w.dist, w.seed, r,
                            first=first, sigma=w.sigma) for r in range(w.P)]


def oracle_full(w, bufs, op=None):
    """Run the oracle in place over full host buffers of workload w."""
    return orc.allreduce(bufs, op=OPS[op or w.op], kind=KINDS[w.topo], k=w.k, rows=w.rows,
                         cols=w.cols, buckets=w.bucket_list())


def bucket_of(w, e):
    for off, cnt in w.bucket_list():
        if off <= e < off + cnt:
            return off, cnt
    raise IndexError(e)


def oracle_at(w, idx, op=None, dist=None):
    """Expected result at the global element indices idx (identical on every
    rank).  Each bucket is its own all-reduce, so the oracle walks only the
    bucket holding the element, restricted to a one-element window."""
    idx = np.asarray(idx, dtype=np.uint64)
    dt = np_dtype(w.dtype)
    inputs = [synth.gather_host(idx, synth_dtype(w.dtype), dist or w.dist, w.seed, r,
                                sigma=w.sigma) for r in range(w.P)]
    out = np.empty(idx.size, dtype=dt)
    for j, e in enumerate(idx.tolist()):
        off, cnt = bucket_of(w, e)
        one = [np.array([inputs[r][j]], dtype=dt) for r in range(w.P)]
        orc.allreduce(one, op=OPS[op or w.op], kind=KINDS[w.topo], k=w.k, rows=w.rows,
                      cols=w.cols, buckets=[(0, cnt)], window=(e - off, e - off + 1),
                      count_only_n=cnt)
        out[j] = one[0][0]
    return out, inputs


def sample_indices(w, count, seed=0):
    """Random elements plus the edges of every chunk of the first, last and a
    middle bucket (where ragged pieces and tails live)."""
    rng = np.random.default_rng(seed)
    picks = set(rng.integers(0, w.n, count).tolist()) if w.n else set()
    bl = w.bucket_list()
    for off, cnt in [bl[0], bl[len(bl) // 2], bl[-1]]:
        q = 16 // w.esize
        parts = orc.split(cnt, w.k, q) if w.topo == "multiring" else [0, cnt]
        for a, b in zip(parts[:-1], parts[1:]):
            m = w.cols if w.topo == "torus2d" else w.P
            edges = orc.split(b - a, m, q)
            for x in edges:
                for d in (-1, 0, 1):
                    e = off + a + x + d
                    if off <= e < off + cnt:
                        picks.add(e)
    return np.array(sorted(picks), dtype=np.uint64)
