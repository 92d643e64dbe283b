"""fp64 CPU oracle for the activation-sparse FFN decode path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``; never by the product package. It shares no code with the
HIP path. The arithmetic lives in ``oracle.c`` (plain C loops in double); this module only
marshals numpy arrays to it.

Parity is pinned for every function here by the CPU test-suite (closed forms, invariants,
brute force and hand-worked fixtures); the one quantity left unpinned is predictor *quality*
against true activations, which needs trained predictors the pages describe but do not give.
"""
from .oracle import (  # noqa: F401
    F16, F32, F64, build, load, half_to_double, predict, threshold, compact, forward, dense,
    dense_f16act, round_half, preact, profile_counts, permutation, pack_rows, n_hot_for, threads, open_library,
    set_library, OMP_LIB_PATH,
)
