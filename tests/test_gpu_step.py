"""GPU parity of the fused step (swa_rma_step): one launch that appends the token
and attends with it (then the split merge, as in the decode) must leave the same
state and produce the same outputs, bit for bit, as the append followed by the
decode; and both match the oracle's append followed by its decode within the
decode's bars.

Cases: ragged states at a batch that splits the key range and at one that does
not, the window ring wrapping (pos + 1 a multiple of 1024), an empty state, a
full pending block (no token taken), and several steps in a row on one workspace
(its per-sequence counters must return to zero after every call).  The oracle's
state evolves on its own throughout: it never takes a key or value from the GPU.
"""

import numpy as np
import pytest
import torch

import oracle as O
import swa_memory_anchor_amd as R
import synth

from gpu_util import (DEV, assert_attn_close, assert_keys_close, bf16_dev, bits_host, decode_gpu,
                      download, f32_dev, norm_dev, upload)

pytestmark = pytest.mark.gpu

COUNTS = [(1024, 255, 70000), (37, 5, 600), (0, 0, -1), (1000, 254, 1023), (16, 15, 15),
          (1024, 0, 262143), (0, 256, 5000), (513, 128, 2047)]


def _rand_state(tag, counts):
    B = len(counts)
    st = O.new_layer_state(B)
    for nm in ("win_k", "win_v", "bank_k", "bank_v", "pend_k", "pend_v"):
        a = getattr(st, nm)
        a[...] = synth.normal_bf16_np(synth.stream_key(tag, nm), a.size).reshape(a.shape)
    for b, (nb, npd, pos) in enumerate(counts):
        st.n_bank[b], st.n_pend[b], st.pos[b] = nb, npd, pos
    return st


def _gains(tag):
    return {nm: synth.normal_f32_np(synth.stream_key(tag, nm), (256,), 1.0, 0.1)
            for nm in ("gq_win", "gk_win", "gq_rma", "gk_rma")}


def _token(tag, B, t):
    recs = [synth.normal_bf16_np(synth.stream_key(tag, nm, t), B * 1024).reshape(B, 4, 256)
            for nm in ("kw", "vw", "kr", "vr")]
    q = [synth.normal_bf16_np(synth.stream_key(tag, nm, t), B * 4096).reshape(B, 16, 256)
         for nm in ("qw", "qr")]
    score = synth.normal_f32_np(synth.stream_key(tag, "score", t), (B, 4))
    return recs, q, score


def _outs(B):
    return [torch.full((B, 16, 256), 7.0, dtype=torch.bfloat16, device=DEV),
            torch.full((B, 16), 7.0, device=DEV),
            torch.full((B, 16, 256), 7.0, dtype=torch.bfloat16, device=DEV),
            torch.full((B, 16), 7.0, device=DEV)]


def _same(x, y):
    if x.dtype == torch.bfloat16:
        return torch.equal(x.view(torch.int16), y.view(torch.int16))
    return torch.equal(x.view(torch.int32), y.view(torch.int32))


def _assert_states_equal(a: R.LayerState, b: R.LayerState, what):
    for f in ("win_k", "win_v", "bank_k", "bank_v", "pend_k", "pend_v", "bank_score", "bank_src",
              "pend_score", "pend_src", "n_bank", "n_pend", "pos"):
        assert _same(getattr(a, f), getattr(b, f)), f"{what}: {f}"


def _oracle_append(st, recs, g, score):
    """The oracle's append on every sequence whose pending block has room (a full
    block takes no token, as the library documents)."""
    from dataclasses import fields

    for b in range(st.pos.shape[0]):
        if st.n_pend[b] >= st.block:
            continue
        one = O.LayerState(**{f.name: getattr(st, f.name)[b:b + 1] for f in fields(O.LayerState)})
        O.append(one, *[r[b:b + 1] for r in recs], g["gk_win"], g["gk_rma"], 1e-6, 1e7,
                 score=None if score is None else score[b:b + 1])


def _tiled_state(tag, counts, reps):
    """A state of len(counts) * reps sequences whose K/V contents repeat every
    len(counts) sequences (cheaper to draw); the tokens still differ per sequence."""
    from dataclasses import fields

    base = _rand_state(tag, counts)
    return O.LayerState(**{f.name: np.concatenate([getattr(base, f.name)] * reps)
                           for f in fields(O.LayerState)})


def _run_both(tag, counts, steps, with_score, reps=1):
    B = len(counts) * reps
    print(f"case: step {tag} B={B} splits={R.rma_decode_splits(B)} steps={steps} "
          f"score={with_score}", flush=True)
    st = _tiled_state(tag, counts, reps)
    g = _gains(tag)
    nm = norm_dev(g)
    fused, split = upload(st), upload(st)
    ws = R.step_workspace(B)
    for t in range(steps):
        recs, q, score = _token(tag, B, t)
        dev = [bf16_dev(r) for r in recs]
        qd = [bf16_dev(x) for x in q]
        sd = f32_dev(score) if with_score else None
        o_f = _outs(B)
        R.swa_rma_step(fused, B, *dev, sd, *qd, nm, *o_f, ws)
        R.swa_rma_append(split, B, *dev, sd, nm)
        o_s = decode_gpu(split, qd[0], qd[1], nm)
        torch.cuda.synchronize()
        _assert_states_equal(fused, split, f"{tag} t={t}")
        for x, y, nmo in zip(o_f, o_s, ("o_win", "lse_win", "o_rma", "lse_rma")):
            assert _same(x, y), f"{tag} t={t}: {nmo}"
        off = (R.rma_decode_workspace_bytes(B) + 255) // 256 * 256
        assert not ws[off:].any(), "counters not reset"
        # the oracle: append, then decode
        _oracle_append(st, recs, g, score if with_score else None)
        ref = O.decode(st, q[0], q[1], g["gq_win"], g["gq_rma"], 1e-6, 1e7)
        assert_attn_close(bits_host(o_f[0]), o_f[1].cpu().numpy(), ref[0], ref[1],
                          what=f"window t={t}")
        assert_attn_close(bits_host(o_f[2]), o_f[3].cpu().numpy(), ref[2], ref[3],
                          what=f"anchor t={t}")
        got = download(fused)
        for f in ("win_v", "pend_v", "pend_src", "n_pend", "pos", "n_bank"):
            assert np.array_equal(getattr(got, f), getattr(st, f)), f
        if with_score:
            assert np.array_equal(got.pend_score, st.pend_score)
        for f in ("win_k", "pend_k"):
            assert_keys_close(getattr(got, f), getattr(st, f), what=f)
    return download(fused)


@pytest.mark.parametrize("with_score", [True, False])
def test_step_matches_append_then_decode_split_batch(with_score):
    assert R.rma_decode_splits(len(COUNTS)) > 1
    got = _run_both(f"step_split_{with_score}", COUNTS, 3, with_score)
    full = COUNTS.index((0, 256, 5000))
    assert got.n_pend[full] == 256 and got.pos[full] == 5000


def test_step_matches_append_then_decode_unsplit_batch():
    assert R.rma_decode_splits(8 * len(COUNTS)) == 1
    _run_both("step_unsplit", COUNTS, 2, True, reps=8)


def test_step_batch_one_stream_wraps_the_window():
    # pos + 1 = 1024 puts the new key in slot 0; 16 splits at batch 1
    got = _run_both("step_b1", [(700, 250, 1021)], 4, False)
    assert got.pos[0] == 1025 and got.n_pend[0] == 254


def test_step_from_an_empty_state():
    got = _run_both("step_empty", [(0, 0, -1), (0, 0, -1)], 3, True)
    assert list(got.pos) == [2, 2] and list(got.n_pend) == [3, 3]


def test_step_trajectory_with_commits_against_an_independent_oracle():
    """300 fused steps at a ragged batch that splits, with a commit whenever a
    sequence's pending block fills, against the oracle's own append / commit /
    decode chain started from the same state and never synchronised with the GPU."""
    counts = [(1024, 250, 5000), (10, 0, 100), (600, 128, 1500), (0, 0, -1)]
    B = len(counts)
    tag = "step_traj"
    st = _rand_state(tag, counts)
    for b in range(B):
        for g in range(4):
            st.bank_src[b, g] = synth.distinct_ints_np(synth.stream_key(tag, "src", b, g), 1024,
                                                       10**6, 10**6 + 4096)
        st.pend_src[b] = np.arange(256) + 2 * 10**6  # distinct from every appended position
    st.bank_score[...] = synth.normal_f32_np(synth.stream_key(tag, "bs"), st.bank_score.shape)
    st.pend_score[...] = synth.normal_f32_np(synth.stream_key(tag, "ps"), st.pend_score.shape)
    g = _gains(tag)
    nm = norm_dev(g)
    dst = upload(st)
    ws = R.step_workspace(B)
    keep = torch.empty(B, 4, 1024, dtype=torch.int32, device=DEV)
    worst = 0.0
    commits = 0
    for t in range(300):
        if (st.n_pend >= st.block).any():
            R.rma_commit_topk(dst, B, keep)
            torch.cuda.synchronize()
            k_ref = O.commit(st)
            assert np.array_equal(keep.cpu().numpy(), k_ref), f"commit before step {t}"
            commits += 1
        recs, q, score = _token(tag, B, t)
        o = _outs(B)
        R.swa_rma_step(dst, B, *[bf16_dev(r) for r in recs], f32_dev(score),
                       *[bf16_dev(x) for x in q], nm, *o, ws)
        torch.cuda.synchronize()
        _oracle_append(st, recs, g, score)
        if t % 10 == 0 or t > 290:
            ref = O.decode(st, q[0], q[1], g["gq_win"], g["gq_rma"], 1e-6, 1e7)
            rw, _ = assert_attn_close(bits_host(o[0]), o[1].cpu().numpy(), ref[0], ref[1],
                                      what=f"trajectory t={t} window")
            rr, _ = assert_attn_close(bits_host(o[2]), o[3].cpu().numpy(), ref[2], ref[3],
                                      what=f"trajectory t={t} anchor")
            worst = max(worst, float(rw.max()), float(rr.max()))
    got = download(dst)
    for f in ("win_v", "pend_v", "bank_v", "pend_src", "bank_src", "n_pend", "n_bank", "pos"):
        assert np.array_equal(getattr(got, f), getattr(st, f)), f
    assert np.array_equal(got.bank_score.view(np.uint32), st.bank_score.view(np.uint32))
    for f in ("win_k", "pend_k", "bank_k"):
        assert_keys_close(getattr(got, f), getattr(st, f), what=f"trajectory {f}")
    print(f"trajectory: 300 steps, {commits} commits, worst output error {worst:.3e}")
    assert commits >= 2
