"""The fp64 oracle over whole workloads, in a pool of worker processes.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU baseline may use this module; the library never calls it.

The oracle's own functions do the arithmetic: ``prefill_group_rows`` (the
prefill restricted to some query rows of one sequence and one KV group,
pinned against ``prefill``) and ``decode``.  This module only cuts a workload
into independent pieces -- (sequence b, KV group u, rows r0..r1-1) for a
prefill, one sequence for a decode -- and evaluates them in parallel.  Each
worker draws its sequence's inputs itself from the seeded generators of
``synthetic`` (the same values the GPU receives), so no input crosses a
process boundary; results come back as float64 blocks.

Workers are fresh interpreters (the "spawn" start method: a child process is
started, the parent is never replaced) with one BLAS thread each, so the
pool uses exactly as many cores as it has workers.
"""

from __future__ import annotations

import contextlib
import multiprocessing as mp
import os

import numpy as np

from . import gqa_oracle as _orc

# largest score block (query rows x keys, per head) a prefill piece forms
MAX_BLOCK_ELEMS = 1 << 24
MAX_WORKERS = 16
_BLAS_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS",
             "BLIS_NUM_THREADS", "NUMEXPR_NUM_THREADS")


def host_cores() -> int:
    """Cores this process may run on (its CPU affinity), capped at 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_WORKERS))


# ------------------------------------------------------------- workers ---

_CACHE: dict = {}


def _workload(key, overrides):
    import dataclasses
    from synthetic import WORKLOADS
    w = WORKLOADS[key]
    return dataclasses.replace(w, **dict(overrides)) if overrides else w


def _prefill_inputs(key, overrides, b):
    tag = ("prefill", key, overrides, b)
    if tag not in _CACHE:
        from synthetic import gen_prefill_b
        _CACHE.clear()          # one sequence at a time per worker
        _CACHE[tag] = gen_prefill_b(_workload(key, overrides), b)
    return _CACHE[tag]


def _prefill_piece(task):
    key, overrides, b, u, r0, r1, theta = task
    w = _workload(key, overrides)
    q, k, v = _prefill_inputs(key, overrides, b)
    th = w.theta if theta is None else theta
    return b, u, r0, r1, _orc.prefill_group_rows(q, k, v, u, r0, r1, theta=th, scale=w.scale)


def _decode_piece(task):
    key, overrides, b = task
    from synthetic import gen_decode_cache_b, gen_decode_query
    w = _workload(key, overrides)
    q = gen_decode_query(w, B=b + 1)[b:b + 1]
    kc, vc = gen_decode_cache_b(w, b)
    return b, _orc.decode(q, kc[None], vc[None], w.L, w.q_pos, theta=w.theta, scale=w.scale)[0]


# ----------------------------------------------------------------- pool --

@contextlib.contextmanager
def oracle_pool(workers: int | None = None):
    """A spawn-context process pool of ``workers`` (default: host_cores())
    single-threaded workers."""
    n = host_cores() if workers is None else max(1, int(workers))
    saved = {k: os.environ.get(k) for k in _BLAS_ENV}
    for k in _BLAS_ENV:
        os.environ[k] = "1"
    try:
        pool = mp.get_context("spawn").Pool(n)
    finally:
        for k, val in saved.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val
    try:
        yield pool
    finally:
        pool.close()
        pool.join()


def stop_resource_tracker() -> bool:
    """End the helper process that the "spawn" start method keeps for the
    pools' named semaphores, once every pool is closed, so that the caller
    leaves no process behind.  The closed pools are collected first: their
    semaphores unregister through the helper while it still runs.  Closing
    its pipe makes it exit; it is then waited for.  A later pool starts a
    new one.  Returns whether one was running."""
    import gc
    from multiprocessing import resource_tracker
    gc.collect()
    tracker = resource_tracker._resource_tracker
    with tracker._lock:
        fd, pid = tracker._fd, tracker._pid
        if fd is None or pid is None:
            return False
        os.close(fd)
        tracker._fd = None
        tracker._pid = None
        os.waitpid(pid, 0)
    return True


def prefill_tasks(key: str, overrides: tuple = (), rows_per_piece: int = 512,
                  batches=None, groups=None, theta=None):
    """Pieces (b, u, r0, r1) of a prefill workload, the ones with the most
    keys first.  ``overrides``: (field, value) pairs replacing fields of the
    workload (e.g. (("L", 300),) for a shorter draw of the same recipe)."""
    w = _workload(key, overrides)
    n = max(16, min(rows_per_piece, MAX_BLOCK_ELEMS // w.L))
    tasks = []
    for b in (range(w.B) if batches is None else batches):
        for u in (range(w.h_kv) if groups is None else groups):
            for r0 in range(0, w.L, n):
                tasks.append((key, tuple(overrides), b, u, r0, min(r0 + n, w.L), theta))
    tasks.sort(key=lambda t: -t[5])
    return tasks


def prefill_pieces(pool, tasks):
    """Yield (b, u, r0, r1, O[b, r0:r1, heads of u] float64) as they finish."""
    yield from pool.imap_unordered(_prefill_piece, tasks)


def decode_pieces(pool, key: str, overrides: tuple = (), batches=None):
    """Yield (b, O[b] float64 [h_q, d]) of a decode workload as they finish."""
    w = _workload(key, overrides)
    tasks = [(key, tuple(overrides), b) for b in (range(w.B) if batches is None else batches)]
    yield from pool.imap_unordered(_decode_piece, tasks)


class Comparison:
    """Running max-abs and relative-L2 of got (GPU, as float64) against the
    oracle's pieces, over the whole output."""

    def __init__(self):
        self.max_abs = 0.0
        self.err2 = 0.0
        self.ref2 = 0.0
        self.count = 0
        self.worst = None
        self.nonfinite = 0

    def add(self, got, want, where):
        got = np.asarray(got, np.float64)
        diff = got - want
        bad = ~np.isfinite(got)
        self.nonfinite += int(bad.sum())
        m = float(np.max(np.abs(np.where(bad, 0.0, diff)))) if diff.size else 0.0
        if self.worst is None or m > self.max_abs:
            self.max_abs = m
            self.worst = where
        self.err2 += float(np.sum(np.where(bad, 0.0, diff) ** 2))
        self.ref2 += float(np.sum(want * want))
        self.count += diff.size

    @property
    def rel_l2(self) -> float:
        return (self.err2 / self.ref2) ** 0.5 if self.ref2 > 0 else 0.0

    def summary(self) -> str:
        return (f"{self.count} outputs: max-abs {self.max_abs:.3e} (at {self.worst}), "
                f"rel-L2 {self.rel_l2:.3e}, non-finite {self.nonfinite}")
