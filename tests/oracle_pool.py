"""The oracle's decode on every (sequence, layer) unit of a full-size workload, spread
over worker processes.

Each worker regenerates the unit's inputs on the host from the seeded generators
(state, query, gains: the same counter streams the device copies were drawn from),
runs the float64 oracle for both branches (on the dequantised rows for an E4M3 or
INT8 state), and compares with the GPU's outputs for
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
    q = W.q_np(wl, layer, b)
    if wl.extra.get("kv") == "e4m3":  # codes + row scales, dequantised by the FP8 oracle
        from oracle import fp8_ref as F

        rows = {nm: F.dequantize(*W.kv_fp8_np(wl, layer, nm, b)) for nm in W.KV_NAMES}
        dec, pos = F.decode_one, wl.position
    elif wl.extra.get("kv") == "int8":  # codes + row scales, dequantised by the INT8 oracle
        from oracle import fp8_ref as F
        from oracle import int8_ref as I

        rows = {nm: I.dequantize(*W.kv_i8_np(wl, layer, nm, b)) for nm in W.KV_NAMES}
        dec, pos = F.decode_one, wl.position
    else:
        rows = W.decode_state_np(wl, layer, b)
        dec, pos = O.decode_one, rows["pos"]
    ow, lwr = dec(list(rows["win_k"]), list(rows["win_v"]), q, g["gq_win"], pos, wl.eps,
                  wl.rope_base)
    keys = [np.concatenate([rows["bank_k"][gg], rows["pend_k"][gg]]) for gg in range(4)]
    vals = [np.concatenate([rows["bank_v"][gg], rows["pend_v"][gg]]) for gg in range(4)]
    orr, lrr = dec(keys, vals, q, g["gq_rma"], pos, wl.eps, wl.rope_base)
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


_GDN = {}


def gdn_unit_errors(task):
    """task = (workload name, layer, b, new matrices [32][128][128], output bits
    [32][128], convolution ring bits [4][8192]) from the GPU -> (b, layer, largest
    state error / bound, largest output row error, ring bit-exact)."""
    import synth
    from gdn_check import out_rel, state_err_ratio
    from oracle import gdn_ref as G
    from synth import workloads as W

    name, layer, b, s_gpu, o_bits, ring_gpu = task
    wl = W.WORKLOADS[name]
    prm = _GDN.get((name, layer))
    if prm is None:
        prm = _GDN[(name, layer)] = (W.gdn_params(wl, layer), W.gdn_gate_inputs(wl, layer))
    p, (a, bb) = prm
    sdt = np.float16 if wl.extra["state"] == "f16" else np.float32
    st = G.GdnState(np.stack([W.gdn_state_np(wl, layer, b, h) for h in range(32)])[None]
                    .astype(sdt), W.gdn_conv_np(wl, layer, b)[None].copy())
    ref_o = G.decode_step(st, W.gdn_x_np(wl, layer, b)[None], a[b:b + 1], bb[b:b + 1],
                          p["conv_w"], p["a_log"], p["dt_bias"], [wl.position])
    return (b, layer, state_err_ratio(s_gpu, st.S[0]),
            float(out_rel(synth.bf16_bits_to_f32_np(o_bits), ref_o[0]).max()),
            bool(np.array_equal(ring_gpu, st.conv[0])))


def all_gdn_unit_errors(tasks, procs=None):
    import multiprocessing as mp

    procs = procs or workers()
    ctx = mp.get_context("spawn")
    with ctx.Pool(procs, initializer=_init_worker) as pool:
        return pool.map(gdn_unit_errors, tasks, chunksize=max(1, len(tasks) // (8 * procs)))


_SCORER = {}


def score_unit_errors(task):
    """task = (workload name, layer, b, GPU scores [256][4] of sequence b's burst) ->
    (b, largest |s_gpu - s_ref| / max(1, |s_ref|)), the oracle's scorer in float64
    on the host-regenerated hidden rows."""
    import oracle as O
    from synth import workloads as W

    name, layer, b, s_gpu = task
    wl = W.WORKLOADS[name]
    w = _SCORER.get((name, layer))
    if w is None:
        w = _SCORER[(name, layer)] = W.scorer_weights(wl, layer)
    ref = O.score(W.burst_hidden_np(wl, layer, b), *w).astype(np.float64)
    err = np.abs(np.asarray(s_gpu, np.float64) - ref) / np.maximum(1.0, np.abs(ref))
    return (b, float(err.max()))


def all_score_unit_errors(tasks, procs=None):
    import multiprocessing as mp

    procs = procs or workers()
    ctx = mp.get_context("spawn")
    with ctx.Pool(procs, initializer=_init_worker) as pool:
        return pool.map(score_unit_errors, tasks, chunksize=max(1, len(tasks) // (8 * procs)))


def prefill_unit_errors(task):
    """task = (workload name, layer, b, chunk, GPU results of sequence b: o_win bits
    [C][16][256], lse_win [C][16], o_rma bits, lse_rma, pending K and V rows [4][C][256]
    bits, window K and V rows at the chunk's ring slots [4][C][256] bits, n_pend, pos).

    The oracle runs the chunk as C successive (append, decode) steps on the sequence's
    steady-state layer (regenerated from the seeds: full window and bank, empty
    pending block) -> (b, layer, worst output error, worst LSE error, worst key error
    / bound, values and counters exact)."""
    import oracle as O
    from attn_check import attn_errors, key_err_ratio
    from synth import workloads as W

    name, layer, b, C, ow_b, lw, or_b, lr, pk, pv, wk, wv, n_pend, pos = task
    wl = W.WORKLOADS[name]
    g = _GAINS.get((name, layer))
    if g is None:
        g = _GAINS[(name, layer)] = W.gains(wl, layer)
    s = W.decode_state_np(wl, layer, b)
    one = O.new_layer_state(1)
    for nm in W.KV_NAMES:
        getattr(one, nm)[0] = s[nm]
    one.n_bank[0], one.n_pend[0], one.pos[0] = O.BANK, 0, wl.position
    recs = [W.prefill_record_np(wl, layer, nm, b, C) for nm in W.RECORD_NAMES]
    q = W.prefill_q_np(wl, layer, b, C)
    ref = [[], [], [], []]
    for i in range(C):
        O.append(one, *[r[i][None] for r in recs], g["gk_win"], g["gk_rma"], wl.eps,
                 wl.rope_base)
        d = O.decode(one, q[i][None], q[i][None], g["gq_win"], g["gq_rma"], wl.eps, wl.rope_base)
        for j in range(4):
            ref[j].append(d[j][0])
    r1, e1 = attn_errors(ow_b, lw, np.stack(ref[0]), np.stack(ref[1]))
    r2, e2 = attn_errors(or_b, lr, np.stack(ref[2]), np.stack(ref[3]))
    slots = (wl.position + 1 + np.arange(C)) % O.WINDOW
    kerr = max(key_err_ratio(pk, one.pend_k[0][:, :C]), key_err_ratio(wk, one.win_k[0][:, slots]))
    exact = (np.array_equal(pv, one.pend_v[0][:, :C]) and
             np.array_equal(wv, one.win_v[0][:, slots]) and
             int(n_pend) == int(one.n_pend[0]) and int(pos) == int(one.pos[0]))
    return (b, layer, float(max(r1.max(), r2.max())), float(max(e1.max(), e2.max())), kerr, exact)


def all_prefill_unit_errors(tasks, procs=None):
    import multiprocessing as mp

    procs = procs or workers()
    ctx = mp.get_context("spawn")
    with ctx.Pool(procs, initializer=_init_worker) as pool:
        return pool.map(prefill_unit_errors, tasks, chunksize=1)
