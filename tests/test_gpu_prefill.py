"""GPU parity of the chunked prefill against the oracle's token-by-token steps.

swa_rma_prefill(C tokens) is defined as C successive append + decode steps; the
oracle runs exactly those steps one token at a time (oracle.append then
oracle.decode) and every output row and the final state are compared.
"""

import numpy as np
import pytest
import torch

import oracle as O
import swa_memory_anchor_amd as R
import synth
from synth import workloads as W

from gpu_util import (DEV, assert_attn_close, assert_keys_close, bf16_dev, bits_host, download,
                      f32_dev, norm_dev, upload)

pytestmark = pytest.mark.gpu


def _state(tag, counts):
    B = len(counts)
    st = O.new_layer_state(B)
    for nm in ("win_k", "win_v", "bank_k", "bank_v", "pend_k", "pend_v"):
        a = getattr(st, nm)
        a[...] = synth.normal_bf16_np(synth.stream_key(tag, nm), a.size).reshape(a.shape)
    for b, (nb, npd, pos) in enumerate(counts):
        st.n_bank[b], st.n_pend[b], st.pos[b] = nb, npd, pos
        # sources only order equal scores; keep them distinct from every position the
        # test appends (and non-negative, as the ABI requires)
        for g in range(4):
            st.bank_src[b, g] = synth.distinct_ints_np(synth.stream_key(tag, "src", b, g), 1024,
                                                       10**6, 10**6 + 4096)
        st.pend_src[b] = np.arange(256) + 2 * 10**6
    return st


def _gains(tag):
    return {nm: synth.normal_f32_np(synth.stream_key(tag, nm), (256,), 1.0, 0.1)
            for nm in ("gq_win", "gk_win", "gq_rma", "gk_rma")}


def _run(tag, counts, C, same_q=True):
    B = len(counts)
    st = _state(tag, counts)
    g = _gains(tag)
    recs = [synth.normal_bf16_np(synth.stream_key(tag, "rec", i), B * C * 1024).reshape(B, C, 4, 256)
            for i in range(4)]
    qw = synth.normal_bf16_np(synth.stream_key(tag, "qw"), B * C * 4096).reshape(B, C, 16, 256)
    qr = qw if same_q else synth.normal_bf16_np(synth.stream_key(tag, "qr"),
                                                B * C * 4096).reshape(B, C, 16, 256)
    score = synth.normal_f32_np(synth.stream_key(tag, "score"), (B, C, 4))
    dst = upload(st)
    nm = norm_dev(g)
    o_w = torch.full((B, C, 16, 256), 3.0, dtype=torch.bfloat16, device=DEV)
    o_r = torch.full_like(o_w, 3.0)
    l_w = torch.full((B, C, 16), 3.0, device=DEV)
    l_r = torch.full_like(l_w, 3.0)
    qwd = bf16_dev(qw)
    qrd = qwd if same_q else bf16_dev(qr)
    R.swa_rma_prefill(dst, B, C, *[bf16_dev(r) for r in recs], f32_dev(score), qwd, qrd, nm,
                      o_w, l_w, o_r, l_r, R.prefill_workspace(B, C))
    torch.cuda.synchronize()
    got = download(dst)
    ow, lw, orr, lr = bits_host(o_w), l_w.cpu().numpy(), bits_host(o_r), l_r.cpu().numpy()
    for b, (nb, npd, pos) in enumerate(counts):
        if npd + C > 256:
            # no room in the pending block: untouched, empty outputs
            for k in ("win_k", "win_v", "pend_k", "pend_v", "n_pend", "pos", "pend_src"):
                assert np.array_equal(getattr(got, k)[b], getattr(st, k)[b]), k
            assert np.all(ow[b] == 0) and np.all(np.isneginf(lw[b]))
            continue
        one = O.new_layer_state(1)
        for k in one.__dict__:
            getattr(one, k)[...] = getattr(st, k)[b:b + 1]
        ref_w, ref_lw, ref_r, ref_lr = [], [], [], []
        for i in range(C):
            O.append(one, *[r[b:b + 1, i] for r in recs], g["gk_win"], g["gk_rma"], 1e-6, 1e7,
                     score=score[b:b + 1, i])
            d = O.decode(one, qw[b:b + 1, i], qr[b:b + 1, i], g["gq_win"], g["gq_rma"], 1e-6, 1e7)
            ref_w.append(d[0][0])
            ref_lw.append(d[1][0])
            ref_r.append(d[2][0])
            ref_lr.append(d[3][0])
        assert_attn_close(ow[b], lw[b], np.stack(ref_w), np.stack(ref_lw), what=f"b={b} win")
        assert_attn_close(orr[b], lr[b], np.stack(ref_r), np.stack(ref_lr), what=f"b={b} rma")
        for k in ("win_v", "pend_v", "pend_src", "n_pend", "pos", "bank_k", "n_bank"):
            assert np.array_equal(getattr(got, k)[b], getattr(one, k)[0]), (b, k)
        assert np.array_equal(got.pend_score[b].view(np.uint32), one.pend_score[0].view(np.uint32))
        for k in ("win_k", "pend_k"):
            assert_keys_close(getattr(got, k)[b], getattr(one, k)[0], what=f"b={b} {k}")


def test_prefill_ragged_states_and_chunk():
    # first chunk of an empty stream; ring partly filled with unaligned pending;
    # steady state filling the block exactly; a sequence with no room
    counts = [(0, 0, -1), (300, 20, 500), (1024, 56, 70000), (1024, 100, 9000)]
    _run("prefill_a", counts, C=200)


@pytest.mark.parametrize("C", [1, 16, 37, 256])
def test_prefill_chunk_sizes(C):
    counts = [(1024, 0, 65535), (513, 0, 1100)]
    _run(f"prefill_c{C}", counts, C, same_q=(C != 37))


def test_prefill_then_decode_continues_the_stream():
    # prefill a block, commit, then one decode step: same as doing it token by token
    B, C = 2, 256
    tag = "prefill_stream"
    counts = [(1024, 0, 40959), (200, 0, 455)]
    st = _state(tag, counts)
    g = _gains(tag)
    recs = [synth.normal_bf16_np(synth.stream_key(tag, "rec", i), B * (C + 1) * 1024).reshape(
        B, C + 1, 4, 256) for i in range(4)]
    q = synth.normal_bf16_np(synth.stream_key(tag, "q"), B * (C + 1) * 4096).reshape(B, C + 1, 16, 256)
    score = synth.normal_f32_np(synth.stream_key(tag, "score"), (B, C, 4))
    dst = upload(st)
    nm = norm_dev(g)
    outs = [torch.empty(B, C, 16, 256, dtype=torch.bfloat16, device=DEV), torch.empty(B, C, 16, device=DEV),
            torch.empty(B, C, 16, 256, dtype=torch.bfloat16, device=DEV), torch.empty(B, C, 16, device=DEV)]
    qd = bf16_dev(np.ascontiguousarray(q[:, :C]))
    R.swa_rma_prefill(dst, B, C, *[bf16_dev(np.ascontiguousarray(r[:, :C])) for r in recs],
                      f32_dev(score), qd, qd, nm, *outs, R.prefill_workspace(B, C))
    keep = torch.empty(B, 4, 1024, dtype=torch.int32, device=DEV)
    R.rma_commit_topk(dst, B, keep)
    R.swa_rma_append(dst, B, *[bf16_dev(np.ascontiguousarray(r[:, C])) for r in recs], None, nm)
    o = [torch.empty(B, 16, 256, dtype=torch.bfloat16, device=DEV), torch.empty(B, 16, device=DEV),
         torch.empty(B, 16, 256, dtype=torch.bfloat16, device=DEV), torch.empty(B, 16, device=DEV)]
    qd1 = bf16_dev(np.ascontiguousarray(q[:, C]))
    R.swa_rma_decode_attn(dst, B, qd1, qd1, nm, *o, R.decode_workspace(B))
    torch.cuda.synchronize()
    ref = st.copy()
    for i in range(C):
        O.append(ref, *[r[:, i] for r in recs], g["gk_win"], g["gk_rma"], 1e-6, 1e7, score=score[:, i])
    k_ref = O.commit(ref)
    assert np.array_equal(keep.cpu().numpy(), k_ref)
    O.append(ref, *[r[:, C] for r in recs], g["gk_win"], g["gk_rma"], 1e-6, 1e7)
    d = O.decode(ref, q[:, C], q[:, C], g["gq_win"], g["gq_rma"], 1e-6, 1e7)
    assert_attn_close(bits_host(o[0]), o[1].cpu().numpy(), d[0], d[1], what="next win")
    assert_attn_close(bits_host(o[2]), o[3].cpu().numpy(), d[2], d[3], what="next rma")


def test_prefill_b512_full_size_sampled_sequences():
    """The full-size prefill_b512 call (512 sequences x 256 tokens, steady-state layer)
    in the benchmark's launch configuration: sampled sequences replayed token by token
    by the oracle in worker processes (all 256 output rows of both branches, the
    chunk's stored keys and values, the counters); every output row finite."""
    import oracle_pool

    wl = W.PREFILL_B512
    B, C = wl.batch, 256
    out = {}
    for layer in (0, 5):
        print(f"case: {wl.name} layer={layer} B={B} C={C}", flush=True)
        st = R.alloc_layer_state(B, DEV, zero_kv=False)
        for nm in W.KV_NAMES:
            W.kv_torch_(wl, layer, nm, getattr(st, nm))
        meta = W.decode_meta(wl, layer)
        meta["n_pend"][:] = 0
        for k, v in meta.items():
            getattr(st, k).copy_(torch.from_numpy(v).to(DEV))
        nm_ = norm_dev(W.gains(wl, layer), wl.eps, wl.rope_base)
        recs = []
        for nm in W.RECORD_NAMES:
            t = torch.empty(B, C, 4, 256, dtype=torch.bfloat16, device=DEV)
            W.prefill_record_torch_(wl, layer, nm, t)
            recs.append(t)
        q = torch.empty(B, C, 16, 256, dtype=torch.bfloat16, device=DEV)
        W.prefill_q_torch_(wl, layer, q)
        o_w = torch.empty(B, C, 16, 256, dtype=torch.bfloat16, device=DEV)
        o_r = torch.empty_like(o_w)
        l_w = torch.empty(B, C, 16, device=DEV)
        l_r = torch.empty_like(l_w)
        R.swa_rma_prefill(st, B, C, *recs, None, q, q, nm_, o_w, l_w, o_r, l_r,
                          R.prefill_workspace(B, C))
        torch.cuda.synchronize()
        for x in (o_w, o_r, l_w, l_r):
            assert torch.isfinite(x.float()).all()
        rng = np.random.default_rng(256 + layer)
        picks = sorted(set(int(x) for x in rng.integers(0, B, 12)) | {0, B - 1})
        slots = torch.from_numpy((wl.position + 1 + np.arange(C)) % O.WINDOW).to(DEV)
        for b in picks:
            out[(layer, b)] = (bits_host(o_w[b]), l_w[b].cpu().numpy(), bits_host(o_r[b]),
                               l_r[b].cpu().numpy(), bits_host(st.pend_k[b, :, :C]),
                               bits_host(st.pend_v[b, :, :C]),
                               bits_host(st.win_k[b].index_select(1, slots)),
                               bits_host(st.win_v[b].index_select(1, slots)),
                               int(st.n_pend[b]), int(st.pos[b]))
        del st, recs, q, o_w, o_r, l_w, l_r
    tasks = [(wl.name, layer, b, C, *v) for (layer, b), v in out.items()]
    print(f"checking {len(tasks)} sequences x {C} tokens against the oracle", flush=True)
    res = oracle_pool.all_prefill_unit_errors(tasks)
    for b, layer, o_err, l_err, k_err, exact in res:
        print(f"layer {layer} b={b}: out {o_err:.3e} lse {l_err:.3e} keys {k_err:.3f} "
              f"exact={exact}")
    assert all(r[5] for r in res), "stored values or counters differ"
    assert max(r[2] for r in res) <= 2e-2 and max(r[3] for r in res) <= 2e-2
    assert max(r[4] for r in res) <= 1.0
