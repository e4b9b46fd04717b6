"""Worker side of the full-size parity tests: the CPU oracle on one
(sequence, head) at a time, in a pool of separate processes (spawned, so they
never touch the GPU), compared with the GPU outputs handed over with it.

Imports only NumPy and the oracle.  Each worker runs single-threaded BLAS so
that the pool, not the BLAS, spreads the work over the host cores."""
from __future__ import annotations

import os

import numpy as np

import oracle

ATOL_REL = 2e-2  # |gpu - ref| <= ATOL_REL * (1 + |ref|), elementwise


def init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass


def pool_size() -> int:
    """At most 15 workers (the host share of one GPU is 16 cores)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return max(1, min(15, cores))


def compare_head(task):
    """task = (b, h, n, bias_mode, bias_arg, inputs, gpu): inputs q, k, v, dO
    and gpu outputs O, dQ, dK, dV, each [n, d] float32 (exact copies of the
    16-bit values).  Returns (b, h, n, {output: worst ratio})."""
    b, h, n, bias_mode, bias_arg, inputs, gpu = task
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in inputs)
    ref = oracle.head(q, k, v, do, n, bias_mode=bias_mode, bias_arg=bias_arg)
    ratios = {}
    for name, g, r in zip(("o", "dq", "dk", "dv"), gpu, ref):
        g = np.asarray(g, dtype=np.float64)
        ratios[name] = float(np.max(np.abs(g - r) / (ATOL_REL * (1.0 + np.abs(r))))) if r.size else 0.0
    return b, h, n, ratios
