"""Every kernel variant the tuning knobs select gives the oracle's bits.

The knobs (ddl_set_tuning) change launch shapes and instruction order only:
load batch, broadcast ranks per workgroup, non-temporal loads, tile
anchoring, the reduce kernel's loop order.  Each setting is run on small cases with ragged chunks (ring,
multi-ring, torus; binary32 and binary16) and compared bit for bit with the
oracle's walk.
"""
import numpy as np
import pytest

import sgd_gradient_all_amd as ddl
from synth.workloads import Workload

from _helpers import ddl_topo, host_inputs, oracle_full, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    Workload("ring-P40", 40, 50_021, "f32", "mean", "ring", dist="normal", sigma=1e-2, seed=61,
             buckets=[(20_000, 30_021), (0, 20_000)]),
    Workload("torus-4x4-f16", 16, 70_003, "f16", "mean", "torus2d", rows=4, cols=4,
             dist="normal", sigma=1e-2, seed=62),
    Workload("mring-P12-k3", 12, 33_337, "f32", "sum", "multiring", k=3, dist="uniform",
             seed=63),
]

SETTINGS = ([("fused_batch", b) for b in (2, 4, 8)] +
            [("reduce_batch", b) for b in (1, 2, 8)] +
            [("bcast_ranks", g) for g in (1, 3, 100)] +
            [("bcast_tiles", t) for t in (2, 5)] +
            [("bcast_xcd", 8), ("bcast_xcd", 3)] +
            [("reduce_nt_load", 0), ("fused_nt_load_max_p", 1000), ("anchor", 1),
             ("anchor", 2)] +
            # the reduce kernel rank by rank at every rank count, and tile
            # by tile at every rank count
            [("reduce_ranks_min_p", 0), ("reduce_ranks_min_p", 1000)] +
            # the broadcast's store wait off and on for both element types
            [("bcast_store_wait", 0), ("bcast_store_wait", 1)] +
            [("fused_store_wait", 0), ("fused_store_wait", 1)])


@pytest.fixture(autouse=True)
def restore_defaults():
    yield
    for k in ddl._ddl.TUNE:
        ddl.set_tuning(k, -1)


@pytest.fixture(scope="module")
def expected():
    out = {}
    for w in CASES:
        g = host_inputs(w)
        ref = [x.copy() for x in g]
        oracle_full(w, ref)
        out[w.name] = (g, ref)
    return out


@pytest.mark.parametrize("knob,value", SETTINGS, ids=lambda v: str(v))
def test_knob_setting_is_bitwise(knob, value, expected):
    ddl.set_tuning(knob, value)
    for w in CASES:
        g, ref = expected[w.name]
        for passes in (1, 2):
            say(f"case tuning {knob}={value} {w.name} passes={passes}")
            bufs = [torch.from_numpy(x).cuda() for x in g]
            plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), w.bucket_list(), "fused")
            plan.set_fused_passes(passes)
            plan.execute(bufs)
            torch.cuda.synchronize()
            plan.destroy()
            for r in (0, 1, w.P - 1):
                got = bufs[r].cpu().numpy()
                assert got.tobytes() == ref[r].tobytes(), (knob, value, w.name, passes, r)
    # the step kernels read the anchoring knob too
    if knob == "anchor":
        w = CASES[0]
        g, ref = expected[w.name]
        bufs = [torch.from_numpy(x).cuda() for x in g]
        plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), w.bucket_list(), "stepwise")
        plan.set_step_form(1)   # the per-step kernels' tiles
        plan.execute(bufs)
        torch.cuda.synchronize()
        plan.destroy()
        assert all(bufs[r].cpu().numpy().tobytes() == ref[r].tobytes() for r in (0, w.P - 1))


@pytest.mark.parametrize("batch", [2, 4, 8])
def test_sgd_load_batch_is_bitwise(batch):
    """The SGD variant of the one-kernel pass under every load batch."""
    import oracle as orc
    from _helpers import oracle_full
    ddl.set_tuning("fused_batch", batch)
    for w in CASES:
        say(f"case tuning sgd fused_batch={batch} {w.name}")
        g = host_inputs(w)
        y = [x.copy() for x in g]
        oracle_full(w, y)
        rng = np.random.default_rng(w.seed)
        w0 = [rng.standard_normal(w.n).astype(np.float32) for _ in range(w.P)]
        want = [x.copy() for x in w0]
        orc.sgd(want, y[0], 0.03)
        bufs = [torch.from_numpy(x).cuda() for x in g]
        weights = [torch.from_numpy(x).cuda() for x in w0]
        plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), w.bucket_list(), "fused")
        plan.execute_sgd(bufs, weights, 0.03, keep_grads=True)
        torch.cuda.synchronize()
        plan.destroy()
        for r in (0, w.P - 1):
            assert weights[r].cpu().numpy().tobytes() == want[r].tobytes(), (batch, w.name, r)
            assert bufs[r].cpu().numpy().tobytes() == y[r].tobytes(), (batch, w.name, r)
