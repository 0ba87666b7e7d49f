"""Worker processes for running the CPU oracle over many independent query heads or rows in the
parity tests. The oracle's functions are called unchanged; only the units of work are split.

The pool forks the test process, so the workers see the caller's arrays without copying them.
They run numpy only and never touch the GPU (forked children of a process that has initialised
the GPU must not use it), and they leave through os._exit, so no GPU runtime teardown runs in
them. At most 8 workers: with the parent that stays well inside the box's limit on processes
that hold the GPU device open.
"""
from __future__ import annotations

import multiprocessing as mp
import os

_JOB = None


def n_workers(cap: int = 8) -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def _run(i):
    fn, items = _JOB
    return fn(items[i])


def pmap(fn, items, workers: int | None = None):
    """[fn(x) for x in items], the calls spread over forked worker processes. fn may be a closure:
    the workers inherit it (and everything it refers to) through the fork."""
    global _JOB
    items = list(items)
    nw = min(workers or n_workers(), max(1, len(items)))
    if nw == 1:
        return [fn(x) for x in items]
    _JOB = (fn, items)
    try:
        with mp.get_context("fork").Pool(nw) as pool:
            return pool.map(_run, range(len(items)), chunksize=1)
    finally:
        _JOB = None


tmap = pmap
