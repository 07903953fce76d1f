"""GPU parity of the FP8 K/V state entry points (E4M3 codes + one FP32 scale per
row) against ``oracle.fp8_ref``.

Decode runs on states drawn directly as stored codes and scales; append is checked
code for code (values bit-exact, keys within the E4M3 bound their FP32 rounding
allows); commit is bit-exact; a short stream (append -> commit -> decode) ties
the three together; the full-size workload is checked on sampled units.
"""

import numpy as np
import pytest
import torch

from oracle import fp8_ref as F
import swa_memory_anchor_amd as R
import synth
from synth import core as C
from synth import workloads as W

import oracle_pool
from gpu_util import (ATTN_TOL, DEV, KV, KV_SCALES, assert_attn_close, assert_fp8_keys_close,
                      bf16_dev, bits_host, decode_gpu_fp8, download_fp8, f32_dev, norm_dev, upload_fp8)

pytestmark = pytest.mark.gpu


def _rand_state(tag, counts):
    """FP8 oracle state: N(0,1)-like E4M3 codes, scales in [3/512, 4/512), and the
    given (n_bank, n_pend, pos) per sequence."""
    st = F.new_layer_state_fp8(len(counts))
    for nm in KV:
        a = getattr(st, nm)
        a[...] = C.normal_e4m3_np(synth.stream_key(tag, nm), a.size).reshape(a.shape)
        s = getattr(st, nm + "s")
        s[...] = C.row_scale_np(synth.stream_key(tag, nm, "s"), s.size).reshape(s.shape)
    for b, (nb, npd, pos) in enumerate(counts):
        st.n_bank[b], st.n_pend[b], st.pos[b] = nb, npd, pos
    return st


def _gains(tag):
    return {nm: synth.normal_f32_np(synth.stream_key(tag, nm), (256,), 1.0, 0.1)
            for nm in ("gq_win", "gk_win", "gq_rma", "gk_rma")}


COUNTS = [(1024, 256, 70000), (37, 5, 600), (0, 1, 0), (1000, 255, 1023), (16, 16, 15),
          (1024, 0, 262143), (0, 0, -1), (513, 129, 1024)]


@pytest.mark.parametrize("same_q", [True, False])
def test_fp8_decode_ragged_multi_split(same_q):
    print(f"case: fp8 decode ragged batch={len(COUNTS)} same_q={same_q}", flush=True)
    st = _rand_state("fp8_dec", COUNTS)
    B = len(COUNTS)
    g = _gains("fp8_dec")
    qw = synth.normal_bf16_np(synth.stream_key("fp8_dec", "qw"), B * 4096).reshape(B, 16, 256)
    qr = qw if same_q else synth.normal_bf16_np(synth.stream_key("fp8_dec", "qr"),
                                                B * 4096).reshape(B, 16, 256)
    dst = upload_fp8(st)
    qwd = bf16_dev(qw)
    qrd = qwd if same_q else bf16_dev(qr)
    assert R.rma_decode_splits(B) > 1
    o_w, l_w, o_r, l_r = decode_gpu_fp8(dst, qwd, qrd, norm_dev(g))
    torch.cuda.synchronize()
    ref = F.decode(st, qw, qr, g["gq_win"], g["gq_rma"], 1e-6, 1e7)
    assert_attn_close(bits_host(o_w), l_w.cpu().numpy(), ref[0], ref[1], what="fp8 window")
    assert_attn_close(bits_host(o_r), l_r.cpu().numpy(), ref[2], ref[3], what="fp8 anchor")
    b_empty = COUNTS.index((0, 0, -1))
    assert np.all(bits_host(o_r)[b_empty] == 0) and np.all(np.isneginf(l_r.cpu().numpy()[b_empty]))
    assert np.all(np.isneginf(l_w.cpu().numpy()[b_empty]))
    after = download_fp8(dst)
    for nm in KV + KV_SCALES:
        assert np.array_equal(getattr(after, nm), getattr(st, nm)), nm


def test_fp8_decode_zero_scale_rows_and_extreme_codes():
    """Rows of an all-zero input (scale 0, codes 0) and rows of +-448 codes."""
    counts = [(64, 32, 5000), (1024, 256, 99999)]
    st = _rand_state("fp8_edge", counts)
    st.win_k[0, 1, :100] = 0
    st.win_ks[0, 1, :100] = 0.0
    st.bank_v[1, 2, :50] = 0x7E  # +448
    st.bank_v[1, 2, 50:100] = 0xFE  # -448
    st.pend_k[1, 3, :10] = 0x7E
    st.pend_ks[1, 3, :10] = 1.0 / 448  # decodes to 1.0 per element: the row's scores peak
    B = len(counts)
    g = _gains("fp8_edge")
    q = synth.normal_bf16_np(synth.stream_key("fp8_edge", "q"), B * 4096).reshape(B, 16, 256)
    qd = bf16_dev(q)
    o_w, l_w, o_r, l_r = decode_gpu_fp8(upload_fp8(st), qd, qd, norm_dev(g))
    torch.cuda.synchronize()
    ref = F.decode(st, q, q, g["gq_win"], g["gq_rma"], 1e-6, 1e7)
    assert_attn_close(bits_host(o_w), l_w.cpu().numpy(), ref[0], ref[1], what="fp8 edge window")
    assert_attn_close(bits_host(o_r), l_r.cpu().numpy(), ref[2], ref[3], what="fp8 edge anchor")


def test_fp8_append_codes_and_scales():
    print("case: fp8 append", flush=True)
    counts = [(0, 0, -1), (10, 255, 5000), (1024, 100, 1023), (3, 7, 262142)]
    st = _rand_state("fp8_app", counts)
    B = len(counts)
    g = _gains("fp8_app")
    recs = [synth.normal_bf16_np(synth.stream_key("fp8_app", nm), B * 1024).reshape(B, 4, 256)
            for nm in ("kw", "vw", "kr", "vr")]
    # one all-zero value row (half of it -0) and one all-zero key row: scale 0, +0 codes
    recs[1][2, 1] = 0
    recs[1][2, 1, ::2] = 0x8000
    recs[2][1, 3] = 0
    score = synth.normal_f32_np(synth.stream_key("fp8_app", "score"), (B, 4))
    dst = upload_fp8(st)
    nm = norm_dev(g)
    R.swa_rma_append_fp8(dst, B, *[bf16_dev(r) for r in recs], f32_dev(score), nm)
    torch.cuda.synchronize()
    F.append(st, *recs, g["gk_win"], g["gk_rma"], 1e-6, 1e7, score=score)
    got = download_fp8(dst)
    for k in ("win_v", "pend_v", "win_vs", "pend_vs", "pend_score", "pend_src", "n_pend", "pos",
              "bank_k", "bank_ks", "bank_v", "bank_vs"):
        a, b_ = getattr(got, k), getattr(st, k)
        assert np.array_equal(a.view(np.uint8), b_.view(np.uint8)), k
    for k in ("win_k", "pend_k"):
        assert_fp8_keys_close(getattr(got, k), getattr(got, k + "s"), getattr(st, k),
                              getattr(st, k + "s"), what=k)
    assert got.pend_ks[1, 3, 255] == 0.0 and np.all(got.pend_k[1, 3, 255] == 0)
    assert got.win_vs[2, 1, 0] == 0.0 and np.all(got.win_v[2, 1, 0] == 0)
    # a full pending block is left untouched
    st2 = _rand_state("fp8_app_full", [(1024, 256, 9000)])
    d2 = upload_fp8(st2)
    R.swa_rma_append_fp8(d2, 1, *[bf16_dev(r[:1]) for r in recs], None, nm)
    torch.cuda.synchronize()
    g2 = download_fp8(d2)
    assert g2.n_pend[0] == 256 and g2.pos[0] == 9000
    assert np.array_equal(g2.win_k, st2.win_k) and np.array_equal(g2.win_ks, st2.win_ks)


def _commit_state(tag, counts, special=True):
    st = _rand_state(tag, [(nb, npd, 50000 + b) for b, (nb, npd) in enumerate(counts)])
    rng = synth.rng_np(synth.stream_key(tag, "commit"))
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0], np.float32)
    for b in range(len(counts)):
        for g in range(4):
            st.bank_src[b, g] = rng.permutation(40000)[:1024]
            st.bank_score[b, g] = rng.standard_normal(1024).astype(np.float32) * 0.3
        st.pend_src[b] = np.arange(40000, 40256) + rng.integers(0, 5)
        st.pend_score[b] = rng.standard_normal((256, 4)).astype(np.float32) * 0.3
        if special:
            m = rng.random((4, 1024)) < 0.2
            st.bank_score[b][m] = rng.choice(vals, size=int(m.sum()))
            m2 = rng.random((256, 4)) < 0.2
            st.pend_score[b][m2] = rng.choice(vals, size=int(m2.sum()))
            st.bank_score[b, 1, 7] = np.nan
            st.pend_score[b, 3, 2] = np.nan
    return st


COMMIT_COUNTS = [(1024, 256), (1000, 200), (500, 256), (0, 256), (1024, 0), (3, 1), (768, 256),
                 (0, 0), (1023, 1)]


@pytest.mark.parametrize("special", [True, False])
def test_fp8_commit_bit_exact(special):
    print(f"case: fp8 commit special={special}", flush=True)
    st = _commit_state(f"fp8_commit{special}", COMMIT_COUNTS, special)
    dst = upload_fp8(st)
    B = len(COMMIT_COUNTS)
    keep = torch.full((B, 4, 1024), -9, dtype=torch.int32, device=DEV)
    R.rma_commit_topk_fp8(dst, B, keep)
    torch.cuda.synchronize()
    ref_keep = F.commit(st)
    got = download_fp8(dst)
    assert np.array_equal(keep.cpu().numpy(), ref_keep)
    for k in ("bank_k", "bank_v", "bank_src", "n_bank", "n_pend"):
        assert np.array_equal(getattr(got, k), getattr(st, k)), k
    for k in ("bank_ks", "bank_vs", "bank_score"):
        assert np.array_equal(getattr(got, k).view(np.uint32), getattr(st, k).view(np.uint32)), k
    for k in ("pend_k", "pend_v", "pend_ks", "pend_vs", "pend_score", "pend_src"):
        assert np.array_equal(getattr(got, k).view(np.uint8), getattr(st, k).view(np.uint8)), k


def test_fp8_short_stream_append_commit_decode():
    """Two sequences stream 600 tokens (two commits and a partial block) with
    generator-supplied candidate scores, then decode; the GPU state and outputs
    follow the oracle's."""
    T, B = 600, 2
    print(f"case: fp8 stream B={B} T={T}", flush=True)
    tag = "fp8_stream"
    g = _gains(tag)
    nm = norm_dev(g)
    recs = [synth.normal_bf16_np(synth.stream_key(tag, r), T * B * 1024).reshape(T, B, 4, 256)
            for r in ("kw", "vw", "kr", "vr")]
    scores = synth.normal_f32_np(synth.stream_key(tag, "score"), (T, B, 4), 0.0, W.SCORE_STD)
    ref = F.new_layer_state_fp8(B)
    dev = R.alloc_layer_state_fp8(B, DEV)
    recs_d = [bf16_dev(r) for r in recs]
    scores_d = f32_dev(scores)
    for t in range(T):
        if t and t % R.BLOCK == 0:
            R.rma_commit_topk_fp8(dev, B)
            F.commit(ref)
        R.swa_rma_append_fp8(dev, B, *[r[t] for r in recs_d], scores_d[t], nm)
        F.append(ref, *[r[t] for r in recs], g["gk_win"], g["gk_rma"], 1e-6, 1e7,
                 score=scores[t])
    torch.cuda.synchronize()
    got = download_fp8(dev)
    for k in ("bank_src", "pend_src", "n_bank", "n_pend", "pos", "win_v", "win_vs", "bank_v",
              "bank_vs", "pend_v", "pend_vs"):
        assert np.array_equal(getattr(got, k).view(np.uint8), getattr(ref, k).view(np.uint8)), k
    for k in ("win_k", "bank_k", "pend_k"):
        assert_fp8_keys_close(getattr(got, k), getattr(got, k + "s"), getattr(ref, k),
                              getattr(ref, k + "s"), what=k)
    q = synth.normal_bf16_np(synth.stream_key(tag, "q"), B * 4096).reshape(B, 16, 256)
    qd = bf16_dev(q)
    o_w, l_w, o_r, l_r = decode_gpu_fp8(dev, qd, qd, nm)
    torch.cuda.synchronize()
    out = F.decode(ref, q, q, g["gq_win"], g["gq_rma"], 1e-6, 1e7)
    assert_attn_close(bits_host(o_w), l_w.cpu().numpy(), out[0], out[1], what="stream window")
    assert_attn_close(bits_host(o_r), l_r.cpu().numpy(), out[2], out[3], what="stream anchor")


def test_headline_b512_fp8_decode():
    """The full-size FP8 workload in the launch configuration the benchmark times,
    every (sequence, layer) unit checked against the FP8 oracle (worker processes)."""
    wl = W.HEADLINE_B512_FP8
    B, L = wl.batch, wl.layers
    print(f"case: {wl.name} B={B} L={L} splits={R.rma_decode_splits(B)}", flush=True)
    states, qs, norms, gains = [], [], [], []
    for layer in range(L):
        st = R.alloc_layer_state_fp8(B, DEV)
        for nmk in W.KV_NAMES:
            W.kv_fp8_torch_(wl, layer, nmk, getattr(st, nmk), getattr(st, nmk + "s"))
        for k, v in W.decode_meta(wl, layer).items():
            getattr(st, k).copy_(torch.from_numpy(v).to(DEV))
        q = torch.empty(B, 16, 256, dtype=torch.bfloat16, device=DEV)
        W.q_torch_(wl, layer, q)
        gl = W.gains(wl, layer)
        states.append(st)
        qs.append(q)
        gains.append(gl)
        norms.append(norm_dev(gl, wl.eps, wl.rope_base))
    torch.cuda.synchronize()
    outs = [decode_gpu_fp8(states[l], qs[l], qs[l], norms[l]) for l in range(L)]
    torch.cuda.synchronize()
    print("decode done; checking every unit", flush=True)
    rng = np.random.default_rng(5128)
    samples = [(int(b), int(l)) for b, l in zip(rng.integers(0, B, 8), rng.integers(0, L, 8))]
    for b, layer in samples + [(0, 0), (B - 1, L - 1)]:
        # the device copies were drawn from the same counter streams
        codes, scales = W.kv_fp8_np(wl, layer, "bank_k", b)
        assert np.array_equal(states[layer].bank_k[b].cpu().numpy(), codes)
        assert np.array_equal(states[layer].bank_ks[b].cpu().numpy(), scales)
    host = [(bits_host(o_w), l_w.cpu().numpy(), bits_host(o_r), l_r.cpu().numpy())
            for o_w, l_w, o_r, l_r in outs]
    tasks = [(wl.name, layer, b, host[layer][0][b], host[layer][1][b], host[layer][2][b],
              host[layer][3][b]) for layer in range(L) for b in range(B)]
    res = oracle_pool.all_unit_errors(tasks)
    worst = max(res, key=lambda r: max(r[2], r[4]))
    print(f"{wl.name}: all {len(res)} units against the FP8 oracle; worst row-relative error "
          f"{max(worst[2], worst[4]):.3e} (b={worst[0]} layer={worst[1]}), worst lse error "
          f"{max(max(r[3], r[5]) for r in res):.3e}", flush=True)
    bad = [r for r in res if not (max(r[2], r[4]) <= ATTN_TOL and max(r[3], r[5]) <= ATTN_TOL)]
    assert not bad, f"{len(bad)} units out of bound, e.g. {bad[:4]}"
    for o_w, l_w, o_r, l_r in outs:
        assert torch.isfinite(l_w).all() and torch.isfinite(l_r).all()
        assert torch.isfinite(o_w.float()).all() and torch.isfinite(o_r.float()).all()
