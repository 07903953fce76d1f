"""The worker pool that checks every unit of a full-size workload: a unit whose
outputs are the oracle's own (rounded to BF16 as the GPU stores them) passes, and a
planted 5% error in one output row is reported."""

import numpy as np

import oracle as O
from synth import workloads as W

import oracle_pool


def _oracle_outputs(wl, layer, b):
    s = W.decode_state_np(wl, layer, b)
    q = W.q_np(wl, layer, b)
    g = W.gains(wl, layer)
    ow, lw = O.decode_one(list(s["win_k"]), list(s["win_v"]), q, g["gq_win"], s["pos"], wl.eps,
                          wl.rope_base)
    keys = [np.concatenate([s["bank_k"][gg], s["pend_k"][gg]]) for gg in range(4)]
    vals = [np.concatenate([s["bank_v"][gg], s["pend_v"][gg]]) for gg in range(4)]
    orr, lr = O.decode_one(keys, vals, q, g["gq_rma"], s["pos"], wl.eps, wl.rope_base)
    return ow, lw, orr, lr


def test_pool_passes_the_oracles_own_outputs_and_reports_a_planted_error():
    wl = W.STEADY_B64
    tasks = []
    for layer, b in ((0, 0), (7, 63)):
        ow, lw, orr, lr = _oracle_outputs(wl, layer, b)
        ow_bits = O.f64_to_bf16(ow)
        if b == 63:
            bad = ow.copy()
            bad[5] *= 1.05
            ow_bits = O.f64_to_bf16(bad)
        tasks.append((wl.name, layer, b, ow_bits, lw.astype(np.float32), O.f64_to_bf16(orr),
                      lr.astype(np.float32)))
    res = oracle_pool.all_unit_errors(tasks, procs=2)
    (b0, l0, r1, e1, r2, e2), (b1, l1, s1, f1, s2, f2) = res
    assert (b0, l0, b1, l1) == (0, 0, 63, 7)
    assert max(r1, r2) <= 2.0 ** -8 and max(e1, e2) <= 1e-6
    assert 0.04 <= s1 <= 0.06 and s2 <= 2.0 ** -8 and max(f1, f2) <= 1e-6


def test_gdn_pool_passes_the_oracles_own_step_and_reports_a_planted_error():
    from oracle import gdn_ref as G

    wl = W.GDN_DECODE_B512
    layer = 1
    p = W.gdn_params(wl, layer)
    a, bb = W.gdn_gate_inputs(wl, layer)
    tasks = []
    for b in (0, 300):
        st = G.GdnState(np.stack([W.gdn_state_np(wl, layer, b, h) for h in range(32)])[None],
                        W.gdn_conv_np(wl, layer, b)[None].copy())
        o = G.decode_step(st, W.gdn_x_np(wl, layer, b)[None], a[b:b + 1], bb[b:b + 1],
                          p["conv_w"], p["a_log"], p["dt_bias"], [wl.position])
        S = st.S[0].copy()
        ring = st.conv[0].copy()
        if b == 300:  # one matrix element off by 1% and one ring entry changed
            S[3, 5, 7] = np.float16(float(S[3, 5, 7]) * 1.01 + 0.01)
            ring[2, 100] ^= 1
        tasks.append((wl.name, layer, b, S, O.f64_to_bf16(o[0]), ring))
    (b0, _, s0, o0, r0), (b1, _, s1, o1, r1) = oracle_pool.all_gdn_unit_errors(tasks, procs=2)
    assert (b0, b1) == (0, 300)
    assert s0 == 0.0 and o0 <= 2.0 ** -8 and r0
    assert s1 > 10.0 and o1 <= 2.0 ** -8 and not r1


def test_scorer_pool_passes_the_oracles_scores_and_reports_a_planted_error():
    wl = W.COMMIT_BURST_B512
    w1, w2 = W.scorer_weights(wl, 5)
    good = O.score(W.burst_hidden_np(wl, 5, 3), w1, w2)
    bad = good.copy()
    bad[17, 2] = bad[17, 2] * (1 + 3e-5) + 3e-5
    res = oracle_pool.all_score_unit_errors([(wl.name, 5, 3, good), (wl.name, 5, 3, bad)], procs=2)
    assert res[0] == (3, 0.0)
    assert 2e-5 < res[1][1] < 1e-4


def test_prefill_pool_replays_the_chunk_and_reports_a_planted_error():
    """A 3-token chunk on a prefill_b512 sequence: the oracle's own results pass; a
    changed pending value is reported."""
    wl = W.PREFILL_B512
    layer, b, C = 0, 7, 3
    s = W.decode_state_np(wl, layer, b)
    g = W.gains(wl, layer)
    one = O.new_layer_state(1)
    for nm in W.KV_NAMES:
        getattr(one, nm)[0] = s[nm]
    one.n_bank[0], one.n_pend[0], one.pos[0] = O.BANK, 0, wl.position
    recs = [W.prefill_record_np(wl, layer, nm, b, C) for nm in W.RECORD_NAMES]
    q = W.prefill_q_np(wl, layer, b, C)
    outs = [[], [], [], []]
    for i in range(C):
        O.append(one, *[r[i][None] for r in recs], g["gk_win"], g["gk_rma"], wl.eps, wl.rope_base)
        d = O.decode(one, q[i][None], q[i][None], g["gq_win"], g["gq_rma"], wl.eps, wl.rope_base)
        for j in range(4):
            outs[j].append(d[j][0])
    slots = (wl.position + 1 + np.arange(C)) % O.WINDOW
    res_args = [O.f64_to_bf16(np.stack(outs[0])), np.stack(outs[1]).astype(np.float32),
                O.f64_to_bf16(np.stack(outs[2])), np.stack(outs[3]).astype(np.float32),
                one.pend_k[0][:, :C].copy(), one.pend_v[0][:, :C].copy(),
                one.win_k[0][:, slots].copy(), one.win_v[0][:, slots].copy(), C,
                wl.position + C]
    bad = list(res_args)
    bad[5] = bad[5].copy()
    bad[5][1, 2, 3] ^= 0x40
    res = oracle_pool.all_prefill_unit_errors(
        [(wl.name, layer, b, C, *res_args), (wl.name, layer, b, C, *bad)], procs=2)
    (_, _, o0, l0, k0, x0), (_, _, o1, l1, k1, x1) = res
    assert o0 <= 2.0 ** -8 and l0 <= 1e-6 and k0 == 0.0 and x0
    assert o1 <= 2.0 ** -8 and not x1
