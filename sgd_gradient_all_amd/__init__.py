"""Gradient all-reduce (ring, multi-ring, 2D torus) for MI355X.

A thin ctypes binding of libddl.so with the C ABI's names; every step of the
all-reduce runs in the library's HIP kernels.  Buffers may be given as raw
device pointers (int) or as objects with data_ptr() (torch tensors);
streams and events as raw handles or torch objects.
"""
from ._ddl import (  # noqa: F401
    DDL_F32, DDL_F16, DDL_SUM, DDL_MEAN, DDL_RING, DDL_MULTIRING, DDL_TORUS2D,
    DDL_STEPWISE, DDL_FUSED, DDL_K_REDUCE, DDL_K_GATHER, DDL_K_FUSED, DDL_K_FUSED_REDUCE,
    DDL_K_BROADCAST, DDL_K_LARS_NORM, DDL_K_LARS_RATE, DDL_K_UPDATE, DDL_K_WALK, DDL_MAX_RANKS,
    LARS_COEFF, LARS_EPS, DDLError, Plan, ReadyEvent, ddl_allreduce, ddl_cache_clear, ddl_cache_count,
    ddl_plan_create, ddl_strerror, get_tuning, lib, set_tuning, topo,
)
