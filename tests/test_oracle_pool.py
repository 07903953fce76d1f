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
