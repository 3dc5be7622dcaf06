"""Process-parallel oracle quantisation of large weights (test infrastructure).

The NF4 + double-quantisation format splits a flat weight array into groups
of 256 blocks of 64 (16384 weights) that are quantised independently: a
group's codes, block constants and group constant depend on that group's
weights only. So the oracle applied to group-aligned slices, with the
results concatenated, is the oracle applied to the whole array; this module
only runs those slices in worker processes (the oracle's arithmetic is not
touched). A CPU test checks the equality on a ragged array.
"""

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

import oracle

GROUP = 64 * 256


def workers():
    return max(1, min(16, os.cpu_count() or 1))


def make_pool():
    return cf.ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn"))


def quantize_slices(pool, slices):
    """oracle.quantize_nf4_dq of each group-aligned slice (list of arrays)."""
    return list(pool.map(oracle.quantize_nf4_dq, slices))


def quantize_parallel(w32, pool=None):
    """oracle.quantize_nf4_dq(w32), computed on group-aligned slices in parallel."""
    w = np.ascontiguousarray(w32, dtype=np.float32).ravel()
    n = w.size
    ng = -(-n // GROUP)
    chunks = max(1, min(ng, 4 * workers()))
    per = -(-ng // chunks)
    bounds = [(a, min(n, a + per * GROUP)) for a in range(0, n, per * GROUP)]
    if len(bounds) == 1:
        return oracle.quantize_nf4_dq(w)
    own = pool is None
    pool = pool or make_pool()
    try:
        parts = quantize_slices(pool, [w[a:b] for a, b in bounds])
    finally:
        if own:
            pool.shutdown()
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(3))
