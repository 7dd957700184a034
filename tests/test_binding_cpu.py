"""The Python binding's own host logic, without a GPU: a Plan dropped while
its work is in flight is destroyed later instead of leaking its device
tables, streams and events."""
import ctypes
import gc

from sgd_gradient_all_amd import _ddl


class FakeLib:
    """Stands in for libddl.so: ddl_plan_destroy answers DDL_E_BUSY while
    `busy` holds, every call is recorded."""

    def __init__(self):
        self.busy = True
        self.destroyed = []

    def ddl_plan_destroy(self, h):
        v = h.value if isinstance(h, ctypes.c_void_p) else int(h)
        if self.busy:
            return -7
        self.destroyed.append(v)
        return 0

    def ddl_plan_create(self, out, *args):
        out._obj.value = 0x5000
        return 0


def test_plan_dropped_while_busy_is_destroyed_later(monkeypatch):
    fake = FakeLib()
    monkeypatch.setattr(_ddl, "_lib", fake)
    monkeypatch.setattr(_ddl, "_pending", [])
    p = _ddl.Plan.__new__(_ddl.Plan)
    p.handle = ctypes.c_void_p(0x1000)
    del p
    gc.collect()
    assert [h.value for h in _ddl._pending] == [0x1000]
    # still busy: a new plan's creation retries and keeps it
    q = _ddl.Plan(4, 64)
    assert len(_ddl._pending) == 1 and fake.destroyed == []
    # the work completes: the next creation destroys it
    fake.busy = False
    r = _ddl.Plan(4, 64)
    assert _ddl._pending == [] and fake.destroyed == [0x1000]
    # so does an explicit destroy of the live ones, and the exit hook finds
    # nothing left
    q.destroy()
    r.destroy()
    assert fake.destroyed == [0x1000, 0x5000, 0x5000]
    assert _ddl._reap() == 0


def test_exit_hook_retries_pending_handles(monkeypatch):
    fake = FakeLib()
    monkeypatch.setattr(_ddl, "_lib", fake)
    monkeypatch.setattr(_ddl, "_pending", [ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)])
    assert _ddl._reap() == 2
    fake.busy = False
    assert _ddl._reap() == 0
    assert fake.destroyed == [0x2000, 0x3000]
