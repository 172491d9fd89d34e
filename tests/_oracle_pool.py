"""Runs the oracle's key-wise backward over query-row ranges in separate
processes and adds the partial sums (test infrastructure).

A 64K-token head needs every query row's own forward before any key's dK or
dV is known: a full forward of the head in float64.  The rows split into
independent ranges (a key's gradients are sums over rows), so fresh
interpreters (spawned, never forked: they must not inherit the parent's GPU
state) each take a range with one BLAS thread, reading the head's inputs
from float32 files (bf16 values are exact in float32)."""

from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

NAMES = ("q1", "k1", "q2", "k2", "v", "dout")


def _part(job):
    folder, keys, lam_args, rows, causal, eps = job
    from threadpoolctl import threadpool_limits

    from oracle import diffattn_oracle as O

    with threadpool_limits(1):
        t = {n: np.load(os.path.join(folder, n + ".npy"), mmap_mode="r") for n in NAMES}
        return O.backward_dkv_keys(t["q1"], t["k1"], t["q2"], t["k2"], t["v"], keys, *lam_args, t["dout"],
                                   eps=eps, causal=causal, rows=rows)


def dkv_keys(folder, head, keys, lam_args, causal=True, eps=1e-5, rows_per_job=2048, workers=None):
    """dK1, dK2, dV of ``keys`` for one head.  ``head``: name -> float32 array
    ([N, d] or [N, 2d]); written under ``folder``.  lam_args: (lq1, lk1, lq2,
    lk2, lambda_init)."""
    for n in NAMES:
        np.save(os.path.join(folder, n + ".npy"), np.ascontiguousarray(head[n], dtype=np.float32))
    N = head["q1"].shape[0]
    keys = np.asarray(keys)
    start = int(keys.min()) if causal else 0
    jobs = [(folder, keys, lam_args, (r, min(N, r + rows_per_job)), causal, eps)
            for r in range(start, N, rows_per_job)]
    # longest ranges (the last rows, which see the most keys) first
    jobs.reverse()
    n = workers or min(16, len(os.sched_getaffinity(0)))
    # a worker that dies raises BrokenProcessPool here instead of hanging
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn")) as pool:
        parts = list(pool.map(_part, jobs))
    return tuple(sum(p[i] for p in parts) for i in range(3))
