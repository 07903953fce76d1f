"""Oracle work of the batch-1 long-stream test, spread over worker processes.

Two kinds of task, both on the host with NumPy, the oracle and the generators only
(no torch, no GPU; started with "spawn"):

* ``chain_task``: one layer's incremental commit chain over every 256-token block,
  fed the scores the GPU scorer wrote, compared with the GPU's keep_idx commit by
  commit; it also records the cut margins, checks the GPU scores against the
  oracle's scorer on sampled blocks, and there counts the segments whose selection
  would change under the oracle's own scores (a diagnostic).  It returns the bank
  (scores and sources) after the commits that the attention tasks start from.
* ``attn_task``: the oracle's state at the start of one block, rebuilt from the
  seeds -- the window holds the last 1024 positions, the bank holds the records of
  the chain's sources, the pending block is empty -- then the block's tokens are
  appended one by one and the decode outputs at the checked offsets are compared
  with the GPU's.  Stored rows are written by the oracle's own append.
"""

from __future__ import annotations

import numpy as np

from oracle_pool import _init_worker, workers

WL_NAME = "long_stream_b1"


def _wl():
    from synth import workloads as W

    return W, W.WORKLOADS[WL_NAME]


def _cut_margin(scores, srcs, kk):
    """Gap between the kk-th and (kk+1)-th best score of a segment (inf if no cut)."""
    if scores.size <= kk:
        return np.inf
    s = np.sort(scores.astype(np.float64))[::-1]
    return float(s[kk - 1] - s[kk])


def chain_task(task):
    """task = (layer, GPU scores [NBLK][256][4] f32, GPU keep_idx [NBLK][4][1024] i32,
    blocks whose post-commit bank to return, blocks to score with the oracle) ->
    dict with the mismatching commits, margins, score errors, diagnostic and banks."""
    import oracle as O

    W, wl = _wl()
    layer, scores, keeps, snap_blocks, diag_blocks = task
    nblk = scores.shape[0]
    bs = np.zeros((4, O.BANK), np.float32)
    bsrc = np.zeros((4, O.BANK), np.int32)
    nb = 0
    bad = []
    margins = []
    score_err = 0.0
    diag_diff = 0
    snaps = {}
    w1 = w2 = None
    for c in range(nblk):
        ps = scores[c]
        psrc = np.arange(c * O.BLOCK, (c + 1) * O.BLOCK, dtype=np.int32)
        if c in diag_blocks:
            if w1 is None:
                w1, w2 = W.scorer_weights(wl, layer)
            h = W.stream_hidden_np(wl, layer, c * O.BLOCK, (c + 1) * O.BLOCK)
            ref = O.score(h, w1, w2).astype(np.float64)
            err = np.abs(ps.astype(np.float64) - ref) / np.maximum(1.0, np.abs(ref))
            score_err = max(score_err, float(err.max()))
            for g in range(4):
                k_gpu, _ = O.commit_segment(bs[g], bsrc[g], nb, ps[:, g], psrc, O.BLOCK, O.BANK)
                k_own, _ = O.commit_segment(bs[g], bsrc[g], nb, ref.astype(np.float32)[:, g],
                                            psrc, O.BLOCK, O.BANK)
                diag_diff += int(not np.array_equal(k_gpu, k_own))
        kk = min(O.BANK, nb + O.BLOCK)
        for g in range(4):
            margins.append(_cut_margin(np.concatenate([bs[g, :nb], ps[:, g]]), None, kk))
            ki, moves = O.commit_segment(bs[g], bsrc[g], nb, ps[:, g], psrc, O.BLOCK, O.BANK)
            if not np.array_equal(ki, keeps[c, g]):
                bad.append((c, g))
            for t, s in moves:
                bs[g, s] = ps[t, g]
                bsrc[g, s] = psrc[t]
        nb = kk
        if c in snap_blocks:
            snaps[c] = (bs.copy(), bsrc.copy(), nb)
    m = np.array(margins)
    fin = m[np.isfinite(m)]
    return {"layer": layer, "bad": bad, "commits": nblk * 4,
            "margin_min": float(fin.min()) if fin.size else np.inf,
            "margin_below_1e-5": int((fin <= 1e-5).sum()), "score_err": score_err,
            "diag_segments": 4 * len(diag_blocks), "diag_diff": diag_diff, "snaps": snaps}


def _stored_rows(O, W, wl, layer, gains, positions):
    """The rows the oracle's append writes for tokens at `positions`: window key and
    value, candidate key and value, each [n][4][256] BF16 bits."""
    pos = np.asarray(positions, np.int64)
    n = pos.size
    st = O.new_layer_state(n, window=1, bank=1, block=1)
    st.pos[:] = pos - 1
    recs = [W.record_rows_np(wl, layer, nm, pos) for nm in W.RECORD_NAMES]
    O.append(st, *recs, gains["gk_win"], gains["gk_rma"], wl.eps, wl.rope_base)
    return st.win_k[:, :, 0], st.win_v[:, :, 0], st.pend_k[:, :, 0], st.pend_v[:, :, 0]


def attn_task(task):
    """task = (layer, block c, checked offsets (ascending), bank after commit c-1 as
    (scores [4][1024], sources [4][1024], n_bank) or None for c = 0, GPU outputs at the
    checked offsets: o bits [n][2][16][256], lse [n][2][16]) ->
    (layer, c, number of outputs checked, worst output error, worst LSE error)."""
    import oracle as O
    from attn_check import attn_errors

    W, wl = _wl()
    layer, c, offsets, bank, o_bits, lse = task
    g = W.gains(wl, layer)
    p0 = c * O.BLOCK  # first position of the block
    st = O.new_layer_state(1)
    if p0 > 0:
        wpos = np.arange(max(0, p0 - O.WINDOW), p0)
        wk, wv, _, _ = _stored_rows(O, W, wl, layer, g, wpos)
        slots = wpos % O.WINDOW
        st.win_k[0][:, slots] = wk.transpose(1, 0, 2)
        st.win_v[0][:, slots] = wv.transpose(1, 0, 2)
    if bank is not None:
        bsc, bsrc, nb = bank
        if nb:
            src_all = np.unique(bsrc[:, :nb])
            _, _, ck, cv = _stored_rows(O, W, wl, layer, g, src_all)
            where = {int(s): i for i, s in enumerate(src_all)}
            for gg in range(4):
                idx = np.array([where[int(s)] for s in bsrc[gg, :nb]])
                st.bank_k[0, gg, :nb] = ck[idx, gg]
                st.bank_v[0, gg, :nb] = cv[idx, gg]
            st.bank_score[0] = bsc
            st.bank_src[0] = bsrc
        st.n_bank[0] = nb
    st.pos[0] = p0 - 1
    last = max(offsets)
    recs = [W.record_np(wl, layer, nm, p0, p0 + last + 1) for nm in W.RECORD_NAMES]
    q = W.stream_q_np(wl, layer, p0, p0 + last + 1)
    want = set(offsets)
    worst_o = worst_l = 0.0
    k = 0
    for off in range(last + 1):
        O.append(st, *[r[off:off + 1] for r in recs], g["gk_win"], g["gk_rma"], wl.eps,
                 wl.rope_base)
        if off in want:
            d = O.decode(st, q[off:off + 1], q[off:off + 1], g["gq_win"], g["gq_rma"], wl.eps,
                         wl.rope_base)
            r1, e1 = attn_errors(o_bits[k, 0], lse[k, 0], d[0][0], d[1][0])
            r2, e2 = attn_errors(o_bits[k, 1], lse[k, 1], d[2][0], d[3][0])
            worst_o = max(worst_o, float(r1.max()), float(r2.max()))
            worst_l = max(worst_l, float(e1.max()), float(e2.max()))
            k += 1
    assert k == len(offsets)
    return (layer, c, k, worst_o, worst_l)


def run(chain_tasks, attn_tasks_fn, procs=None):
    """Chain tasks first (their banks feed the attention tasks), then attention tasks."""
    import multiprocessing as mp

    procs = procs or workers()
    ctx = mp.get_context("spawn")
    with ctx.Pool(procs, initializer=_init_worker) as pool:
        chains = pool.map(chain_task, chain_tasks, chunksize=1)
        attn = pool.map(attn_task, attn_tasks_fn(chains), chunksize=1)
    return chains, attn
