"""Checkpoint and resume of a layer's state.

The state's capacity is fixed in advance and allocated once (fluxbbs.com,
"EdgeRock-4B 开源：72 MiB 固定 KV，AIME 82.9 分", section "72 MiB 是怎么算出来的":
window, bank and pending block have hard caps, whatever the length).  So a
checkpoint is a byte copy of the state's arrays, the same size at every position,
and a stream resumed from it must continue exactly as the uninterrupted one.

Here a batch of streams runs through fused steps and commits; at a commit
boundary every array is saved to a file and read back into a fresh allocation;
both copies then take the same 300 tokens (crossing another commit) and must give
bit-identical outputs and end in bit-identical states.
"""

import numpy as np
import pytest
import torch

import oracle as O
import swa_memory_anchor_amd as R
import synth

from gpu_util import DEV, bf16_dev, f32_dev, norm_dev, upload

pytestmark = pytest.mark.gpu

FIELDS = ("win_k", "win_v", "bank_k", "bank_v", "bank_score", "bank_src", "pend_k", "pend_v",
          "pend_score", "pend_src", "n_bank", "n_pend", "pos")


def _tokens(tag, B, t):
    recs = [bf16_dev(synth.normal_bf16_np(synth.stream_key(tag, nm, t), B * 1024)
                     .reshape(B, 4, 256)) for nm in ("kw", "vw", "kr", "vr")]
    q = bf16_dev(synth.normal_bf16_np(synth.stream_key(tag, "q", t), B * 4096).reshape(B, 16, 256))
    score = f32_dev(synth.normal_f32_np(synth.stream_key(tag, "score", t), (B, 4)))
    return recs, q, score


def _run(st, B, nm, tag, t0, n):
    """n fused steps from token t0, committing whenever a pending block is full;
    returns every output and keep_idx, concatenated."""
    ws = R.step_workspace(B)
    outs, keeps = [], []
    for t in range(t0, t0 + n):
        if int(st.n_pend.max()) >= O.BLOCK:
            k = torch.empty(B, 4, 1024, dtype=torch.int32, device=DEV)
            R.rma_commit_topk(st, B, k)
            keeps.append(k)
        recs, q, score = _tokens(tag, B, t)
        o = [torch.empty(B, 16, 256, dtype=torch.bfloat16, device=DEV),
             torch.empty(B, 16, device=DEV),
             torch.empty(B, 16, 256, dtype=torch.bfloat16, device=DEV),
             torch.empty(B, 16, device=DEV)]
        R.swa_rma_step(st, B, *recs, score, q, q, nm, *o, ws)
        outs.append(o)
    torch.cuda.synchronize()
    return outs, keeps


def _save(st, path):
    arrays = {}
    for f in FIELDS:
        t = getattr(st, f)
        arrays[f] = (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy()
    np.savez(path, **arrays)
    return sum(a.nbytes for a in arrays.values())


def _load(path, B):
    st = R.alloc_layer_state(B, DEV, zero_kv=False)
    with np.load(path, allow_pickle=False) as z:
        for f in FIELDS:
            t = getattr(st, f)
            src = torch.from_numpy(z[f]).to(DEV)
            (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).copy_(src)
    return st


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_checkpoint_at_a_commit_boundary_resumes_bit_exactly(tmp_path):
    B, tag = 3, "ckpt"
    st0 = O.new_layer_state(B)
    for f in ("win_k", "win_v", "bank_k", "bank_v", "pend_k", "pend_v"):
        a = getattr(st0, f)
        a[...] = synth.normal_bf16_np(synth.stream_key(tag, f), a.size).reshape(a.shape)
    st0.n_bank[:] = [1024, 300, 0]
    st0.n_pend[:] = [56, 0, 0]
    st0.pos[:] = [70000, 2047, -1]
    st0.bank_score[...] = synth.normal_f32_np(synth.stream_key(tag, "bs"), st0.bank_score.shape)
    for b in range(B):
        for g in range(4):
            st0.bank_src[b, g] = synth.distinct_ints_np(synth.stream_key(tag, "src", b, g), 1024,
                                                        10**6, 10**6 + 4096)
        st0.pend_src[b] = np.arange(256) + 2 * 10**6
    nm = norm_dev({k: synth.normal_f32_np(synth.stream_key(tag, k), (256,), 1.0, 0.1)
                   for k in ("gq_win", "gk_win", "gq_rma", "gk_rma")})
    live = upload(st0)
    # 200 tokens, then a commit: the checkpoint is taken at that boundary
    _run(live, B, nm, tag, 0, 200)
    R.rma_commit_topk(live, B, None)
    torch.cuda.synchronize()
    assert int(live.n_pend.max()) == 0
    path = tmp_path / "layer_state.npz"
    nbytes = _save(live, path)
    assert nbytes == R.rma_layer_state_bytes(B), "a checkpoint is exactly the state's bytes"
    resumed = _load(path, B)
    for f in FIELDS:
        assert torch.equal(_bits(getattr(resumed, f)), _bits(getattr(live, f))), f
    # both continue with the same 300 tokens (another commit at token 456)
    out_a, keep_a = _run(live, B, nm, tag, 200, 300)
    out_b, keep_b = _run(resumed, B, nm, tag, 200, 300)
    assert len(keep_a) == len(keep_b) >= 1
    for ka, kb in zip(keep_a, keep_b):
        assert torch.equal(ka, kb)
    for t, (oa, ob) in enumerate(zip(out_a, out_b)):
        for x, y in zip(oa, ob):
            assert torch.equal(_bits(x), _bits(y)), f"token {200 + t}"
    for f in FIELDS:
        assert torch.equal(_bits(getattr(resumed, f)), _bits(getattr(live, f))), f
    # the size of a checkpoint does not depend on the position reached
    assert _save(live, tmp_path / "later.npz") == nbytes
    print(f"checkpoint: {nbytes} bytes for {B} sequences; 300 tokens after resume bit-identical")
