"""GPU parity at a batch whose state offsets pass 2^31 and 2^32 elements.

One layer at B = 4100: a K array is 4100 x 4 x 1024 x 256 BF16 elements (8.6 GB), so
the element offset of sequence b passes 2^31 from b = 2048 and 2^32 from b = 4096; byte
offsets pass 2^31 from b = 1024.  Decode, append, commit and the FP8 decode run over the
whole batch.  Eight sequences on both sides of those boundaries hold seeded contents and
are compared with the oracle; every other sequence holds zero K/V under full, consistent
counts, so the launches have the shape of a full batch.
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import fp8_ref as F
import swa_memory_anchor_amd as R
import synth
from synth import core as C

from gpu_util import (DEV, KV, KV_SCALES, META, assert_attn_close, assert_keys_close, bf16_dev,
                      bits_host, decode_gpu, decode_gpu_fp8, f32_dev, i32_dev, norm_dev)

pytestmark = pytest.mark.gpu

B = 4100
SAMPLE = [0, 1, 1023, 1024, 2047, 2048, 4095, 4099]
# (n_bank, n_pend, pos) of the sampled sequences: partial tiles, empty and full segments
COUNTS = [(1024, 255, 70000), (37, 5, 600), (513, 129, 100), (1024, 0, 262142), (0, 1, 0),
          (16, 16, 15), (700, 200, 5000), (1000, 255, 1023)]


def _gains(tag):
    return {nm: synth.normal_f32_np(synth.stream_key(tag, nm), (256,), 1.0, 0.1)
            for nm in ("gq_win", "gk_win", "gq_rma", "gk_rma")}


def _fill_rest(big):
    """Every sequence outside the sample: full window, bank and pending block, distinct
    sources, zero scores (zero K/V from the allocation)."""
    big.n_bank.fill_(1024)
    big.n_pend.fill_(200)
    big.pos.fill_(70000)
    big.bank_src.copy_(torch.arange(1024, dtype=torch.int32, device=DEV).expand(B, 4, 1024))
    big.pend_src.copy_(torch.arange(100000, 100256, dtype=torch.int32, device=DEV).expand(B, 256))


def _place(big, st, names):
    """Copy the oracle state's rows into the sampled sequences of the device state."""
    idx = torch.tensor(SAMPLE, device=DEV)
    for nm in names:
        a = getattr(st, nm)
        if nm in KV:
            src = bf16_dev(a) if a.dtype == np.uint16 else torch.from_numpy(a).to(DEV)
        else:
            src = f32_dev(a) if a.dtype == np.float32 else i32_dev(a)
        getattr(big, nm)[idx] = src


def _rows(big, nm):
    t = getattr(big, nm)[torch.tensor(SAMPLE, device=DEV)]
    return bits_host(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.fixture(autouse=True)
def _free_device_memory():
    """Each test holds about 39 GB of state; hand it back once the test's frame is gone."""
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_large_batch_decode_then_append():
    print(f"case: decode + append at B={B}, sequences {SAMPLE}", flush=True)
    n = len(SAMPLE)
    st = O.new_layer_state(n)
    for nm in KV:
        a = getattr(st, nm)
        a[...] = synth.normal_bf16_np(synth.stream_key("big", nm), a.size).reshape(a.shape)
    for i, (nb, npd, pos) in enumerate(COUNTS):
        st.n_bank[i], st.n_pend[i], st.pos[i] = nb, npd, pos
    g = _gains("big")
    q = synth.normal_bf16_np(synth.stream_key("big", "q"), n * 4096).reshape(n, 16, 256)
    big = R.alloc_layer_state(B, DEV)
    _fill_rest(big)
    _place(big, st, KV + META)
    idx = torch.tensor(SAMPLE, device=DEV)
    qd = torch.zeros(B, 16, 256, dtype=torch.bfloat16, device=DEV)
    qd[idx] = bf16_dev(q)
    nm = norm_dev(g)
    o_w, l_w, o_r, l_r = decode_gpu(big, qd, qd, nm)
    torch.cuda.synchronize()
    ref = O.decode(st, q, q, g["gq_win"], g["gq_rma"], 1e-6, 1e7)
    assert_attn_close(bits_host(o_w[idx]), l_w[idx].cpu().numpy(), ref[0], ref[1],
                      what=f"window B={B}")
    assert_attn_close(bits_host(o_r[idx]), l_r[idx].cpu().numpy(), ref[2], ref[3],
                      what=f"anchor B={B}")
    # the sequences around them are untouched (zero K/V: uniform softmax over zero rows)
    assert torch.all(o_w[2049:4095].view(torch.int16) == 0)

    recs = [synth.normal_bf16_np(synth.stream_key("big", r), n * 1024).reshape(n, 4, 256)
            for r in ("kw", "vw", "kr", "vr")]
    score = synth.normal_f32_np(synth.stream_key("big", "score"), (n, 4))
    rd = []
    for r in recs:
        t = torch.zeros(B, 4, 256, dtype=torch.bfloat16, device=DEV)
        t[idx] = bf16_dev(r)
        rd.append(t)
    sd = torch.zeros(B, 4, device=DEV)
    sd[idx] = f32_dev(score)
    R.swa_rma_append(big, B, *rd, sd, nm)
    torch.cuda.synchronize()
    O.append(st, *recs, g["gk_win"], g["gk_rma"], 1e-6, 1e7, score=score)
    for nmk in ("win_v", "pend_v", "pend_score", "pend_src", "n_pend", "pos", "bank_k"):
        assert np.array_equal(_rows(big, nmk), getattr(st, nmk)), nmk
    for nmk in ("win_k", "pend_k"):
        assert_keys_close(_rows(big, nmk), getattr(st, nmk), what=f"{nmk} B={B}")


def test_large_batch_commit():
    print(f"case: commit at B={B}, sequences {SAMPLE}", flush=True)
    n = len(SAMPLE)
    st = O.new_layer_state(n)
    rng = synth.rng_np(synth.stream_key("big_commit"))
    for nm in ("bank_k", "bank_v", "pend_k", "pend_v"):
        a = getattr(st, nm)
        a[...] = synth.normal_bf16_np(synth.stream_key("big_commit", nm), a.size).reshape(a.shape)
    for i, (nb, npd, _) in enumerate(COUNTS):
        st.n_bank[i], st.n_pend[i], st.pos[i] = nb, npd, 60000
        for g in range(4):
            st.bank_src[i, g] = rng.permutation(40000)[:1024]
            st.bank_score[i, g] = rng.standard_normal(1024).astype(np.float32) * 0.3
        st.pend_src[i] = np.arange(40000, 40256)
        st.pend_score[i] = rng.standard_normal((256, 4)).astype(np.float32) * 0.3
        st.pend_score[i, 5] = st.bank_score[i, :, 3]  # ties across the two parts
    big = R.alloc_layer_state(B, DEV)
    _fill_rest(big)
    _place(big, st, KV + META)
    keep = torch.full((B, 4, 1024), -9, dtype=torch.int32, device=DEV)
    R.rma_commit_topk(big, B, keep)
    torch.cuda.synchronize()
    ref_keep = O.commit(st)
    assert np.array_equal(keep[torch.tensor(SAMPLE, device=DEV)].cpu().numpy(), ref_keep)
    for nmk in ("bank_k", "bank_v", "bank_src", "n_bank", "n_pend"):
        assert np.array_equal(_rows(big, nmk), getattr(st, nmk)), nmk
    assert np.array_equal(_rows(big, "bank_score").view(np.uint32), st.bank_score.view(np.uint32))
    # a sequence outside the sample: 1024 + 200 equal scores keep the 1024 lowest sources
    # (the bank's own 0..1023) and the counters advance
    assert torch.equal(keep[3000, 0].cpu(), torch.arange(1024, dtype=torch.int32))
    assert int(big.n_bank[3000]) == 1024 and int(big.n_pend[3000]) == 0


def test_large_batch_fp8_decode():
    print(f"case: fp8 decode at B={B}, sequences {SAMPLE}", flush=True)
    n = len(SAMPLE)
    st = F.new_layer_state_fp8(n)
    for nm in KV:
        a = getattr(st, nm)
        a[...] = C.normal_e4m3_np(synth.stream_key("big8", nm), a.size).reshape(a.shape)
        s = getattr(st, nm + "s")
        s[...] = C.row_scale_np(synth.stream_key("big8", nm, "s"), s.size).reshape(s.shape)
    for i, (nb, npd, pos) in enumerate(COUNTS):
        st.n_bank[i], st.n_pend[i], st.pos[i] = nb, npd, pos
    g = _gains("big8")
    q = synth.normal_bf16_np(synth.stream_key("big8", "q"), n * 4096).reshape(n, 16, 256)
    big = R.alloc_layer_state_fp8(B, DEV)
    _fill_rest(big)
    _place(big, st, KV + KV_SCALES + ("n_bank", "n_pend", "pos"))
    idx = torch.tensor(SAMPLE, device=DEV)
    qd = torch.zeros(B, 16, 256, dtype=torch.bfloat16, device=DEV)
    qd[idx] = bf16_dev(q)
    o_w, l_w, o_r, l_r = decode_gpu_fp8(big, qd, qd, norm_dev(g))
    torch.cuda.synchronize()
    ref = F.decode(st, q, q, g["gq_win"], g["gq_rma"], 1e-6, 1e7)
    assert_attn_close(bits_host(o_w[idx]), l_w[idx].cpu().numpy(), ref[0], ref[1],
                      what=f"fp8 window B={B}")
    assert_attn_close(bits_host(o_r[idx]), l_r[idx].cpu().numpy(), ref[2], ref[3],
                      what=f"fp8 anchor B={B}")


def test_large_batch_gdn_step():
    """The GDN step at B = 4100 (FP16 matrices, 4.3 GB: element offsets pass 2^31 from
    sequence 4096) against the oracle on the sampled sequences."""
    from oracle import gdn_ref as G
    from gdn_check import O_TOL, out_rel, state_err_ratio

    print(f"case: gdn step at B={B}, sequences {SAMPLE}", flush=True)
    n = len(SAMPLE)
    st = G.new_state(n, "f16")
    st.S[...] = C.scaled_normal_np(synth.stream_key("big_gdn", "S"), st.S.size,
                                   dtype=np.float16).reshape(st.S.shape)
    st.conv[...] = synth.normal_bf16_np(synth.stream_key("big_gdn", "conv"),
                                        st.conv.size).reshape(st.conv.shape)
    rng = synth.rng_np(synth.stream_key("big_gdn", "params"))
    conv_w = (rng.standard_normal((8192, 4)) * 0.5).astype(np.float32)
    a_log = np.log(rng.uniform(1, 16, 32)).astype(np.float32)
    dt_bias = rng.standard_normal(32).astype(np.float32)
    x = synth.normal_bf16_np(synth.stream_key("big_gdn", "x"), n * 8192).reshape(n, 8192)
    a = (rng.standard_normal((n, 32)) * 2).astype(np.float32)
    bb = (rng.standard_normal((n, 32)) * 2).astype(np.float32)
    pos = np.array([0, 1, 2, 3, 70001, 5, 1023, 262143], np.int32)
    idx = torch.tensor(SAMPLE, device=DEV)
    dev = R.alloc_gdn_state(B, "f16", DEV)
    dev.S[idx] = torch.from_numpy(st.S.copy()).to(DEV)
    dev.conv[idx] = bf16_dev(st.conv)
    xd = torch.zeros(B, 8192, dtype=torch.bfloat16, device=DEV)
    xd[idx] = bf16_dev(x)
    ad = torch.zeros(B, 32, device=DEV)
    ad[idx] = f32_dev(a)
    bd = torch.zeros(B, 32, device=DEV)
    bd[idx] = f32_dev(bb)
    pd = torch.full((B,), 7, dtype=torch.int32, device=DEV)
    pd[idx] = i32_dev(pos)
    o = torch.full((B, 32, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    R.gdn_decode_step(dev, B, xd, ad, bd, pd,
                      R.GdnParams(f32_dev(conv_w), f32_dev(a_log), f32_dev(dt_bias)), o)
    torch.cuda.synchronize()
    ref_o = G.decode_step(st, x, a, bb, conv_w, a_log, dt_bias, pos)
    assert np.array_equal(bits_host(dev.conv[idx]), st.conv), "convolution ring"
    ratio = state_err_ratio(dev.S[idx].cpu().numpy(), st.S)
    assert ratio <= 1.0, f"S out of bound ({ratio:.3f})"
    rel = out_rel(synth.bf16_bits_to_f32_np(bits_host(o[idx])), ref_o)
    print(f"gdn B={B}: state err/bound {ratio:.3f}, out max {rel.max():.3e}")
    assert np.all(np.isfinite(rel)) and rel.max() <= O_TOL


def test_large_batch_prefill():
    """An 8-token chunk for every sequence at B = 4100; the sampled sequences replayed
    token by token by the oracle (those whose pending block has no room are left as
    they were, with empty outputs)."""
    Cn = 8
    print(f"case: prefill C={Cn} at B={B}, sequences {SAMPLE}", flush=True)
    n = len(SAMPLE)
    st = O.new_layer_state(n)
    for nm in KV:
        a = getattr(st, nm)
        a[...] = synth.normal_bf16_np(synth.stream_key("big_pf", nm), a.size).reshape(a.shape)
    # as COUNTS, with the chunk kept inside the 262,144 positions
    counts = [(nb, npd, min(pos, 262144 - 1 - Cn)) for nb, npd, pos in COUNTS]
    for i, (nb, npd, pos) in enumerate(counts):
        st.n_bank[i], st.n_pend[i], st.pos[i] = nb, npd, pos
        for g in range(4):
            st.bank_src[i, g] = synth.distinct_ints_np(synth.stream_key("big_pf", "src", i, g),
                                                       1024, 10**6, 10**6 + 4096)
        st.pend_src[i] = np.arange(256) + 2 * 10**6
    g = _gains("big_pf")
    recs = [synth.normal_bf16_np(synth.stream_key("big_pf", "rec", r), n * Cn * 1024)
            .reshape(n, Cn, 4, 256) for r in range(4)]
    q = synth.normal_bf16_np(synth.stream_key("big_pf", "q"), n * Cn * 4096).reshape(n, Cn, 16, 256)
    score = synth.normal_f32_np(synth.stream_key("big_pf", "score"), (n, Cn, 4))
    big = R.alloc_layer_state(B, DEV)
    _fill_rest(big)
    _place(big, st, KV + META)
    idx = torch.tensor(SAMPLE, device=DEV)

    def spread(x, shape, dtype):
        t = torch.zeros(*shape, dtype=dtype, device=DEV)
        t[idx] = bf16_dev(x) if dtype == torch.bfloat16 else f32_dev(x)
        return t

    rd = [spread(r, (B, Cn, 4, 256), torch.bfloat16) for r in recs]
    qd = spread(q, (B, Cn, 16, 256), torch.bfloat16)
    sd = spread(score, (B, Cn, 4), torch.float32)
    o_w = torch.full((B, Cn, 16, 256), 3.0, dtype=torch.bfloat16, device=DEV)
    o_r = torch.full_like(o_w, 3.0)
    l_w = torch.full((B, Cn, 16), 3.0, device=DEV)
    l_r = torch.full_like(l_w, 3.0)
    R.swa_rma_prefill(big, B, Cn, *rd, sd, qd, qd, norm_dev(g), o_w, l_w, o_r, l_r,
                      R.prefill_workspace(B, Cn))
    torch.cuda.synchronize()
    ow, lw = bits_host(o_w[idx]), l_w[idx].cpu().numpy()
    orr, lr = bits_host(o_r[idx]), l_r[idx].cpu().numpy()
    got = {k: _rows(big, k) for k in KV + META}
    for i, (nb, npd, pos) in enumerate(counts):
        if npd + Cn > 256:
            for k in ("win_k", "win_v", "pend_k", "pend_v", "n_pend", "pos", "pend_src"):
                assert np.array_equal(got[k][i], getattr(st, k)[i]), (i, k)
            assert np.all(ow[i] == 0) and np.all(np.isneginf(lw[i]))
            continue
        one = O.new_layer_state(1)
        for k in one.__dict__:
            getattr(one, k)[...] = getattr(st, k)[i:i + 1]
        ref = [[], [], [], []]
        for t in range(Cn):
            O.append(one, *[r[i:i + 1, t] for r in recs], g["gk_win"], g["gk_rma"], 1e-6, 1e7,
                     score=score[i:i + 1, t])
            d = O.decode(one, q[i:i + 1, t], q[i:i + 1, t], g["gq_win"], g["gq_rma"], 1e-6, 1e7)
            for j in range(4):
                ref[j].append(d[j][0])
        assert_attn_close(ow[i], lw[i], np.stack(ref[0]), np.stack(ref[1]), what=f"seq {i} win")
        assert_attn_close(orr[i], lr[i], np.stack(ref[2]), np.stack(ref[3]), what=f"seq {i} rma")
        for k in ("win_v", "pend_v", "pend_src", "n_pend", "pos", "bank_k", "n_bank"):
            assert np.array_equal(got[k][i], getattr(one, k)[0]), (i, k)
        assert np.array_equal(got["pend_score"][i].view(np.uint32),
                              one.pend_score[0].view(np.uint32))
        for k in ("win_k", "pend_k"):
            assert_keys_close(got[k][i], getattr(one, k)[0], what=f"seq {i} {k}")


def test_large_scorer_call():
    """rma_score over 900,000 rows (4.6 GB of hidden state: row offsets pass 2^31 elements
    from row 838,861) on the 256-row tiles; seeded rows on both sides of that row and at
    the end against the oracle, zero rows scoring exactly zero."""
    from gpu_util import assert_scores_close

    N = 900_000
    rows = [0, 1, 838_860, 838_861, 838_862, 899_743, N - 1]
    print(f"case: scorer N={N}, rows {rows}", flush=True)
    h = synth.normal_bf16_np(synth.stream_key("big_score", "h"), len(rows) * 2560)
    h = h.reshape(len(rows), 2560)
    w1 = synth.normal_f32_np(synth.stream_key("big_score", "w1"), (2560, 256), 0.0, 0.02)
    w2 = synth.normal_f32_np(synth.stream_key("big_score", "w2"), (256, 4), 0.0, 0.02)
    ridx = torch.tensor(rows, device=DEV)
    hd = torch.zeros(N, 2560, dtype=torch.bfloat16, device=DEV)
    hd[ridx] = bf16_dev(h)
    out = torch.full((N, 4), float("nan"), device=DEV)
    R.rma_score(hd, N, 2560, f32_dev(w1), f32_dev(w2), out, 4)
    torch.cuda.synchronize()
    assert_scores_close(out[ridx].cpu().numpy(), O.score(h, w1, w2), what=f"scorer N={N}")
    zero_rows = torch.tensor([2, 838_859, 899_999 - 1], device=DEV)
    assert torch.all(out[zero_rows] == 0)


def test_large_batch_step_equals_append_then_decode():
    """The fused step at B = 4100 gives the bits of append followed by decode: every
    output of the batch, and the appended rows and counters of the sampled sequences."""
    print(f"case: fused step at B={B}", flush=True)
    n = len(SAMPLE)
    st = O.new_layer_state(n)
    for nm in KV:
        a = getattr(st, nm)
        a[...] = synth.normal_bf16_np(synth.stream_key("big_step", nm), a.size).reshape(a.shape)
    for i, (nb, npd, pos) in enumerate(COUNTS):
        st.n_bank[i], st.n_pend[i], st.pos[i] = nb, min(npd, 255), pos
    g = _gains("big_step")
    nm = norm_dev(g)
    idx = torch.tensor(SAMPLE, device=DEV)
    recs = []
    for r in ("kw", "vw", "kr", "vr"):
        t = torch.zeros(B, 4, 256, dtype=torch.bfloat16, device=DEV)
        t[idx] = bf16_dev(synth.normal_bf16_np(synth.stream_key("big_step", r), n * 1024)
                          .reshape(n, 4, 256))
        recs.append(t)
    qd = torch.zeros(B, 16, 256, dtype=torch.bfloat16, device=DEV)
    qd[idx] = bf16_dev(synth.normal_bf16_np(synth.stream_key("big_step", "q"), n * 4096)
                       .reshape(n, 16, 256))
    outs = {}
    for fused in (True, False):
        big = R.alloc_layer_state(B, DEV)
        _fill_rest(big)
        _place(big, st, KV + META)
        o = [torch.empty(B, 16, 256, dtype=torch.bfloat16, device=DEV),
             torch.empty(B, 16, device=DEV),
             torch.empty(B, 16, 256, dtype=torch.bfloat16, device=DEV),
             torch.empty(B, 16, device=DEV)]
        if fused:
            R.swa_rma_step(big, B, *recs, None, qd, qd, nm, *o, R.step_workspace(B))
        else:
            R.swa_rma_append(big, B, *recs, None, nm)
            R.swa_rma_decode_attn(big, B, qd, qd, nm, *o, R.decode_workspace(B))
        torch.cuda.synchronize()
        outs[fused] = ([x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16)
                        for x in o],
                       {k: _rows(big, k) for k in ("win_k", "win_v", "pend_k", "pend_v",
                                                   "n_pend", "pos")})
        del big, o
        torch.cuda.empty_cache()
    for a, b_ in zip(outs[True][0], outs[False][0]):
        assert torch.equal(a, b_)
    for k, v in outs[True][1].items():
        assert np.array_equal(v, outs[False][1][k]), k
