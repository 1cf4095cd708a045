"""Runs the fp64 oracle over many heads in worker processes.

The oracle's causal backward walks a head token by token (about half a second
per head at T = 16384), so checking every head of a full-size workload runs it
in a pool of spawned processes. This module imports only numpy and the oracle:
a spawned worker imports it without torch and never touches the GPU.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import oracle


def workers(limit: int = 16) -> int:
    """Cores this process may use, at most `limit`."""
    return max(1, min(limit, len(os.sched_getaffinity(0))))


def causal_bwd_rows(job):
    """(q, k, v, do, rows, eps, simple, fm) of one decoded head -> the oracle's
    causal dQ, dK, dV on `rows`."""
    q, k, v, do, rows, eps, simple, fm = job
    dq, dk, dv = oracle.causal_bwd_head(q, k, v, do, eps, simple, fm)
    return dq[rows], dk[rows], dv[rows]


def map_heads(fn, jobs, limit: int = 16, timeout: float = 240.0):
    """fn over jobs in spawned worker processes, results in job order; raises
    if the results take longer than `timeout` seconds in all."""
    jobs = list(jobs)
    with ProcessPoolExecutor(max_workers=min(workers(limit), len(jobs)),
                             mp_context=mp.get_context("spawn")) as pool:
        return list(pool.map(fn, jobs, timeout=timeout))
