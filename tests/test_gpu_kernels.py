"""GPU parity of each entry point against the oracle on small, ragged cases.

Sizes span several 16-key tiles with ragged tails, every split path the batch
selects, empty branches, partially filled window/bank/pending blocks, and the
commit's degenerate cases (nothing pending, empty bank, all ties, signed zeros,
NaN scores).
"""

import numpy as np
import pytest
import torch

import oracle as O
import swa_memory_anchor_amd as R
import synth
from synth import workloads as W

from gpu_util import (DEV, assert_attn_close, assert_scores_close, bf16_dev, assert_keys_close,
                      bits_host, decode_gpu, download, f32_dev, norm_dev, upload)

pytestmark = pytest.mark.gpu


def _rand_state(tag, counts):
    """Oracle state with N(0,1) BF16 contents and the given (n_bank, n_pend, pos) per row."""
    B = len(counts)
    st = O.new_layer_state(B)
    for i, nm in enumerate(("win_k", "win_v", "bank_k", "bank_v", "pend_k", "pend_v")):
        a = getattr(st, nm)
        a[...] = synth.normal_bf16_np(synth.stream_key(tag, nm), a.size).reshape(a.shape)
    for b, (nb, npd, pos) in enumerate(counts):
        st.n_bank[b], st.n_pend[b], st.pos[b] = nb, npd, pos
    return st


def _gains(tag):
    return {nm: synth.normal_f32_np(synth.stream_key(tag, nm), (256,), 1.0, 0.1)
            for nm in ("gq_win", "gk_win", "gq_rma", "gk_rma")}


COUNTS = [(1024, 256, 70000), (37, 5, 600), (0, 1, 0), (1000, 255, 1023), (16, 16, 15),
          (1024, 0, 262143), (0, 0, -1), (513, 129, 1024)]


@pytest.mark.parametrize("same_q", [True, False])
def test_decode_ragged_multi_split(same_q):
    print(f"case: decode ragged batch={len(COUNTS)} same_q={same_q}", flush=True)
    st = _rand_state("dec_ragged", COUNTS)
    B = len(COUNTS)
    g = _gains("dec_ragged")
    qw = synth.normal_bf16_np(synth.stream_key("dec_ragged", "qw"), B * 4096).reshape(B, 16, 256)
    qr = qw if same_q else synth.normal_bf16_np(synth.stream_key("dec_ragged", "qr"),
                                                B * 4096).reshape(B, 16, 256)
    dst = upload(st)
    nm = norm_dev(g)
    qwd = bf16_dev(qw)
    qrd = qwd if same_q else bf16_dev(qr)
    assert R.rma_decode_splits(B) > 1
    o_w, l_w, o_r, l_r = decode_gpu(dst, qwd, qrd, nm)
    torch.cuda.synchronize()
    ref = O.decode(st, qw, qr, g["gq_win"], g["gq_rma"], 1e-6, 1e7)
    assert_attn_close(bits_host(o_w), l_w.cpu().numpy(), ref[0], ref[1], what="window")
    assert_attn_close(bits_host(o_r), l_r.cpu().numpy(), ref[2], ref[3], what="anchor")
    # empty branches: o = 0, lse = -inf
    b_empty = COUNTS.index((0, 0, -1))
    assert np.all(bits_host(o_r)[b_empty] == 0) and np.all(np.isneginf(l_r.cpu().numpy()[b_empty]))
    assert np.all(np.isneginf(l_w.cpu().numpy()[b_empty]))
    # the state is read-only for decode
    after = download(dst)
    for nmk in ("win_k", "bank_v", "pend_k"):
        assert np.array_equal(getattr(after, nmk), getattr(st, nmk))


def test_decode_is_deterministic_with_a_reused_workspace():
    B = 4
    st = upload(_rand_state("det", COUNTS[:B]))
    q = bf16_dev(synth.normal_bf16_np(synth.stream_key("det", "q"), B * 4096).reshape(B, 16, 256))
    nm = norm_dev(_gains("det"))
    ws = R.decode_workspace(B)
    assert R.rma_decode_splits(B) > 1 and ws is not None
    outs = []
    for _ in range(3):
        o = [torch.full((B, 16, 256), 7.0, dtype=torch.bfloat16, device=DEV),
             torch.full((B, 16), 7.0, device=DEV),
             torch.full((B, 16, 256), 7.0, dtype=torch.bfloat16, device=DEV),
             torch.full((B, 16), 7.0, device=DEV)]
        R.swa_rma_decode_attn(st, B, q, q, nm, o[0], o[1], o[2], o[3], ws)
        torch.cuda.synchronize()
        outs.append(o)
    for o in outs[1:]:
        for x, y in zip(o, outs[0]):
            assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def test_append_keys_within_derived_bound():
    print("case: append", flush=True)
    counts = [(0, 0, -1), (10, 255, 5000), (1024, 100, 1023), (3, 7, 262142)]
    st = _rand_state("app", counts)
    B = len(counts)
    g = _gains("app")
    recs = [synth.normal_bf16_np(synth.stream_key("app", nm), B * 1024).reshape(B, 4, 256) * 1
            for nm in ("kw", "vw", "kr", "vr")]
    score = synth.normal_f32_np(synth.stream_key("app", "score"), (B, 4))
    dst = upload(st)
    nm = norm_dev(g)
    dev = [bf16_dev(r) for r in recs]
    R.swa_rma_append(dst, B, *dev, f32_dev(score), nm)
    torch.cuda.synchronize()
    O.append(st, *recs, g["gk_win"], g["gk_rma"], 1e-6, 1e7, score=score)
    got = download(dst)
    for nmk in ("win_v", "pend_v", "pend_score", "pend_src", "n_pend", "pos", "bank_k"):
        assert np.array_equal(getattr(got, nmk), getattr(st, nmk)), nmk
    for nmk in ("win_k", "pend_k"):
        assert_keys_close(getattr(got, nmk), getattr(st, nmk), what=nmk)
    # a full pending block is left untouched
    st2 = _rand_state("app_full", [(1024, 256, 9000)])
    d2 = upload(st2)
    R.swa_rma_append(d2, 1, *[bf16_dev(r[:1]) for r in recs], None, nm)
    torch.cuda.synchronize()
    g2 = download(d2)
    assert g2.n_pend[0] == 256 and g2.pos[0] == 9000
    assert np.array_equal(g2.win_k, st2.win_k)


def _score_case(rng, n):
    h = synth.normal_bf16_np(synth.stream_key("score", n), n * 2560).reshape(n, 2560)
    w1 = (0.02 * rng.standard_normal((2560, 256))).astype(np.float32)
    w2 = (0.02 * rng.standard_normal((256, 4))).astype(np.float32)
    return h, w1, w2


@pytest.mark.parametrize("n", [1, 127, 300, 1024])
def test_score_matches_oracle(n):
    print(f"case: score n={n}", flush=True)
    rng = np.random.default_rng(n)
    h, w1, w2 = _score_case(rng, n)
    out = torch.full((n, 4), float("nan"), device=DEV)
    R.rma_score(bf16_dev(h), n, 2560, f32_dev(w1), f32_dev(w2), out, 4)
    torch.cuda.synchronize()
    assert_scores_close(out.cpu().numpy(), O.score(h, w1, w2), what=f"n={n}")


def test_score_strided_output_and_input():
    rng = np.random.default_rng(7)
    h, w1, w2 = _score_case(rng, 200)
    hp = np.zeros((200, 2568), np.uint16)
    hp[:, :2560] = h
    out = torch.full((200, 8), -7.0, device=DEV)
    R.rma_score(bf16_dev(hp), 200, 2568, f32_dev(w1), f32_dev(w2), out, 8)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, 4:] == -7.0)
    assert_scores_close(o[:, :4], O.score(h, w1, w2), what="strided")


def test_score_exact_integer_case_bit_exact():
    # small integers and dyadic weights: every partial sum is exact in FP32 in any
    # order (checked below), so the GPU must reproduce the exact value bit for bit
    rng = np.random.default_rng(8)
    n = 260
    h = rng.integers(-2, 3, size=(n, 2560)).astype(np.float64)
    w1 = rng.integers(-16, 17, size=(2560, 256)) / 64.0
    w2 = rng.integers(-4, 5, size=(256, 4)) / 64.0
    z = h @ w1
    assert (np.abs(h) @ np.abs(w1)).max() * 64 < 2**24
    assert (np.abs(z) @ np.abs(w2)).max() * 4096 < 2**24
    hb = O.f64_to_bf16(h)
    exact = (z @ w2).astype(np.float32)
    out = torch.empty(n, 4, device=DEV)
    R.rma_score(bf16_dev(hb), n, 2560, f32_dev(w1), f32_dev(w2), out, 4)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), exact)
    assert np.array_equal(O.score(hb, w1.astype(np.float32), w2.astype(np.float32)), exact)


def test_score_duplicate_rows_bit_identical():
    rng = np.random.default_rng(9)
    h, w1, w2 = _score_case(rng, 700)
    pairs = [(0, 699), (5, 133), (64, 65), (127, 128), (300, 31), (511, 512)]
    for d, s in pairs:
        h[d] = h[s]
    out = torch.empty(700, 4, device=DEV)
    R.rma_score(bf16_dev(h), 700, 2560, f32_dev(w1), f32_dev(w2), out, 4)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    for d, s in pairs:
        assert np.array_equal(o[d], o[s]), (d, s)


def _commit_state(tag, counts, special=True):
    B = len(counts)
    st = O.new_layer_state(B)
    rng = synth.rng_np(synth.stream_key(tag, "commit"))
    for nm in ("bank_k", "bank_v", "pend_k", "pend_v"):
        a = getattr(st, nm)
        a[...] = synth.normal_bf16_np(synth.stream_key(tag, nm), a.size).reshape(a.shape)
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0], np.float32)
    for b, (nb, npd) in enumerate(counts):
        st.n_bank[b], st.n_pend[b], st.pos[b] = nb, npd, 50000 + b
        for g in range(4):
            st.bank_src[b, g] = rng.permutation(40000)[:1024]
            st.bank_score[b, g] = rng.standard_normal(1024).astype(np.float32) * 0.3
        st.pend_src[b] = np.arange(40000, 40256) + rng.integers(0, 5)
        st.pend_score[b] = rng.standard_normal((256, 4)).astype(np.float32) * 0.3
        if special:
            # ties, signed zeros and NaN scattered over both parts
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
def test_commit_bit_exact(special):
    print(f"case: commit special={special}", flush=True)
    st = _commit_state(f"commit{special}", COMMIT_COUNTS, special)
    dst = upload(st)
    B = len(COMMIT_COUNTS)
    keep = torch.full((B, 4, 1024), -9, dtype=torch.int32, device=DEV)
    R.rma_commit_topk(dst, B, keep)
    torch.cuda.synchronize()
    ref_keep = O.commit(st)
    got = download(dst)
    assert np.array_equal(keep.cpu().numpy(), ref_keep)
    for nmk in ("bank_k", "bank_v", "bank_src", "n_bank", "n_pend"):
        assert np.array_equal(getattr(got, nmk), getattr(st, nmk)), nmk
    assert np.array_equal(got.bank_score.view(np.uint32), st.bank_score.view(np.uint32))
    # pending arrays are not modified
    for nmk in ("pend_k", "pend_v", "pend_score", "pend_src"):
        assert np.array_equal(getattr(got, nmk).view(np.uint8), getattr(st, nmk).view(np.uint8))


def test_commit_all_equal_scores_keep_lowest_sources():
    st = _commit_state("commit_eq", [(1024, 256), (700, 256)], special=False)
    st.bank_score[...] = 0.5
    st.pend_score[...] = 0.5
    dst = upload(st)
    R.rma_commit_topk(dst, 2, None)
    torch.cuda.synchronize()
    ref = st.copy()
    O.commit(ref)
    got = download(dst)
    assert np.array_equal(got.bank_src, ref.bank_src)
    for b, nb in enumerate((1024, 700)):
        n = min(1024, nb + 256)
        assert got.n_bank[b] == n
        for g in range(4):
            cand = np.concatenate([st.bank_src[b, g, :nb], st.pend_src[b]])
            assert np.array_equal(np.sort(got.bank_src[b, g, :n]), np.sort(cand)[:n])


def test_score_large_ragged_uses_big_tiles_and_matches_small_tiles():
    # 33000 rows: 258 tiles of 128 rows (the large-tile kernel) with a ragged tail
    n = 33000
    rng = np.random.default_rng(10)
    h = synth.normal_bf16_np(synth.stream_key("score_big"), n * 2560).reshape(n, 2560)
    w1 = (0.02 * rng.standard_normal((2560, 256))).astype(np.float32)
    w2 = (0.02 * rng.standard_normal((256, 4))).astype(np.float32)
    hd, w1d, w2d = bf16_dev(h), f32_dev(w1), f32_dev(w2)
    out = torch.full((n, 4), float("nan"), device=DEV)
    R.rma_score(hd, n, 2560, w1d, w2d, out, 4)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o))
    rows = np.array([0, 1, 127, 128, 16383, 32767, 32768, 32895, 32999])
    assert_scores_close(o[rows], O.score(h[rows], w1, w2), what="large ragged")
    # the same rows through the small-tile kernel (a 300-row call, 32-row tiles) and the
    # mid-size one (a 17,000-row call, 64-row tiles) give the same bits
    for extra in (291, 16991):
        sub = np.concatenate([rows, np.arange(extra) + 100])
        out2 = torch.empty(len(sub), 4, device=DEV)
        R.rma_score(bf16_dev(h[sub]), len(sub), 2560, w1d, w2d, out2, 4)
        torch.cuda.synchronize()
        assert np.array_equal(out2.cpu().numpy(), o[sub]), len(sub)


def test_score_multi_equals_separate_calls():
    """rma_score_multi: every job's scores are bit-identical to its own rma_score call,
    at a small (32-row tiles) and a mid-size (64-row tiles) row count."""
    rng = np.random.default_rng(77)
    for n in (300, 17000):
        print(f"case: score multi n={n}", flush=True)
        jobs, refs = [], []
        for j in range(3):
            h = bf16_dev(synth.normal_bf16_np(synth.stream_key("score_multi", n, j), n * 2560)
                         .reshape(n, 2560))
            w1 = f32_dev((0.02 * rng.standard_normal((2560, 256))).astype(np.float32))
            w2 = f32_dev((0.02 * rng.standard_normal((256, 4))).astype(np.float32))
            out = torch.full((n, 4), float("nan"), device=DEV)
            ref = torch.empty(n, 4, device=DEV)
            R.rma_score(h, n, 2560, w1, w2, ref, 4)
            jobs.append((h, w1, w2, out))
            refs.append(ref)
        R.rma_score_multi(jobs, n, 2560, 4)
        torch.cuda.synchronize()
        for (_, _, _, out), ref in zip(jobs, refs):
            assert torch.equal(out.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("n_jobs,n,ld_h,ld_s", [(8, 256, 2560, 4), (8, 1, 2560, 4),
                                                 (3, 33, 2568, 8), (8, 1000, 2560, 4),
                                                 (1, 8192, 2560, 4), (1, 8193, 2560, 4),
                                                 (16, 512, 2560, 4), (16, 513, 2560, 4)])
def test_score_multi_ws_equals_single_calls(n_jobs, n, ld_h, ld_s):
    """rma_score_multi_ws: every job's scores are bit-identical to its own rma_score
    call, on the split path (up to 256 row tiles in all, the most jobs included,
    ragged last tile, strided input and output) and past it (8193 rows, or 16 jobs
    of 513: the one-launch path).  The workspace
    starts out holding NaNs, and a second call reuses it."""
    rng = np.random.default_rng(78 + n)
    need = R.rma_score_workspace_bytes(n_jobs, n)
    assert need == (n_jobs * n * 1024 if n_jobs * ((n + 31) // 32) <= 256 else 0)
    print(f"case: score multi ws jobs={n_jobs} n={n} ld={ld_h},{ld_s} ws={need}", flush=True)
    ws = None if need == 0 else torch.full((need // 4,), float("nan"), device=DEV)
    for rep in range(2):
        jobs, refs = [], []
        for j in range(n_jobs):
            h = bf16_dev(synth.normal_bf16_np(synth.stream_key("score_ws", n, j, rep), n * ld_h)
                         .reshape(n, ld_h))
            w1 = f32_dev((0.02 * rng.standard_normal((2560, 256))).astype(np.float32))
            w2 = f32_dev((0.02 * rng.standard_normal((256, 4))).astype(np.float32))
            out = torch.full((n, ld_s), float("nan"), device=DEV)
            ref = torch.full((n, ld_s), float("nan"), device=DEV)
            R.rma_score(h, n, ld_h, w1, w2, ref, ld_s)
            jobs.append((h, w1, w2, out))
            refs.append(ref)
        R.rma_score_multi_ws(jobs, n, ld_h, ld_s, ws)
        torch.cuda.synchronize()
        for (_, _, _, out), ref in zip(jobs, refs):
            assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), rep
            if ld_s > 4:
                assert torch.isnan(out[:, 4:]).all()  # columns past the 4 scores untouched


def test_score_multi_ws_duplicate_rows_and_oracle():
    """Split path: identical rows give identical scores wherever they sit, and the
    scores match the float64 oracle within the scorer's bar."""
    print("case: score multi ws duplicates", flush=True)
    n = 256
    base = synth.normal_bf16_np(synth.stream_key("score_ws_dup"), n * 2560).reshape(n, 2560)
    base[200:] = base[:56]
    rng = np.random.default_rng(5)
    w1 = (0.02 * rng.standard_normal((2560, 256))).astype(np.float32)
    w2 = (0.02 * rng.standard_normal((256, 4))).astype(np.float32)
    out = torch.empty(n, 4, device=DEV)
    ws = R.score_workspace(1, n, DEV)
    R.rma_score_multi_ws([(bf16_dev(base), f32_dev(w1), f32_dev(w2), out)], n, 2560, 4, ws)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.array_equal(o[200:].view(np.uint32), o[:56].view(np.uint32))
    assert_scores_close(o, O.score(base, w1, w2), what="score multi ws")


def test_commit_multi_equals_separate_calls():
    """rma_commit_topk_multi over three layers leaves each state and keep_idx as
    rma_commit_topk does, bit for bit (ragged counts, ties, signed zeros, NaN)."""
    print("case: commit multi", flush=True)
    states = [_commit_state(f"commit_multi_{l}", COMMIT_COUNTS, special=(l != 1)) for l in range(3)]
    B = len(COMMIT_COUNTS)
    multi = [upload(st) for st in states]
    single = [upload(st) for st in states]
    k_multi = [torch.full((B, 4, 1024), -7, dtype=torch.int32, device=DEV) for _ in states]
    k_single = [torch.full((B, 4, 1024), -7, dtype=torch.int32, device=DEV) for _ in states]
    R.rma_commit_topk_multi(multi, B, k_multi)
    for st, k in zip(single, k_single):
        R.rma_commit_topk(st, B, k)
    torch.cuda.synchronize()
    for l in range(3):
        assert torch.equal(k_multi[l], k_single[l]), l
        a, b_ = download(multi[l]), download(single[l])
        for f in ("bank_k", "bank_v", "bank_score", "bank_src", "n_bank", "n_pend", "pos"):
            x, y = getattr(a, f), getattr(b_, f)
            assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                  y.view(np.uint32) if y.dtype == np.float32 else y), (l, f)
