"""The oracle's decode on every (sequence, layer) unit of a full-size workload, spread
over worker processes.

Each worker regenerates the unit's inputs on the host from the seeded generators
(state, query, gains: the same counter streams the device copies were drawn from),
runs the float64 oracle for both branches, and compares with the GPU's outputs for
that unit, which the parent passes in.  Workers import NumPy, the oracle and the
generators only: no torch, no GPU.  They are started with "spawn" (never forked
from a process that holds a GPU context).
"""

from __future__ import annotations

import os

import numpy as np

_GAINS = {}


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def unit_errors(task):
    """task = (workload name, layer, b, o_win bits, lse_win, o_rma bits, lse_rma) ->
    (b, layer, worst output error and worst LSE error of each branch)."""
    import oracle as O
    from attn_check import attn_errors
    from synth import workloads as W

    name, layer, b, ow_bits, lw, or_bits, lr = task
    wl = W.WORKLOADS[name]
    g = _GAINS.get((name, layer))
    if g is None:
        g = _GAINS[(name, layer)] = W.gains(wl, layer)
    s = W.decode_state_np(wl, layer, b)
    q = W.q_np(wl, layer, b)
    ow, lwr = O.decode_one(list(s["win_k"]), list(s["win_v"]), q, g["gq_win"], s["pos"], wl.eps,
                           wl.rope_base)
    keys = [np.concatenate([s["bank_k"][gg], s["pend_k"][gg]]) for gg in range(4)]
    vals = [np.concatenate([s["bank_v"][gg], s["pend_v"][gg]]) for gg in range(4)]
    orr, lrr = O.decode_one(keys, vals, q, g["gq_rma"], s["pos"], wl.eps, wl.rope_base)
    r1, e1 = attn_errors(ow_bits, lw, ow, lwr)
    r2, e2 = attn_errors(or_bits, lr, orr, lrr)
    return (b, layer, float(np.max(r1)), float(np.max(e1)), float(np.max(r2)), float(np.max(e2)))


def workers() -> int:
    """Worker processes: the host's CPU share for one GPU, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def all_unit_errors(tasks, procs=None):
    """unit_errors over every task, in worker processes; results in task order."""
    import multiprocessing as mp

    procs = procs or workers()
    ctx = mp.get_context("spawn")
    with ctx.Pool(procs, initializer=_init_worker) as pool:
        return pool.map(unit_errors, tasks, chunksize=max(1, len(tasks) // (8 * procs)))
