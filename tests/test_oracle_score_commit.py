"""Pins of the oracle's scorer and commit (selection + slot-stable compaction)."""

import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle as O


# ---------------------------------------------------------------- scorer
def _exact_case(rng, n, hidden=2560, mid=256):
    h = rng.integers(-8, 9, size=(n, hidden)).astype(np.float64)
    w1 = rng.integers(-64, 65, size=(hidden, mid)) / 64.0  # multiples of 2^-6, |w| <= 1
    w2 = rng.integers(-64, 65, size=(mid, 4)) / 64.0
    return O.f64_to_bf16(h), w1.astype(np.float32), w2.astype(np.float32), h, w1, w2


def test_score_exact_integer_case_brute_force():
    rng = np.random.default_rng(20)
    hb, w1, w2, h, w1d, w2d = _exact_case(rng, 3, hidden=96, mid=24)
    got = O.score(hb, w1, w2)
    for r in range(3):
        for g in range(4):
            z = [sum(Fraction(int(h[r, k])) * Fraction(w1d[k, j]) for k in range(96))
                 for j in range(24)]
            exact = sum(z[j] * Fraction(w2d[j, g]) for j in range(24))
            assert float(exact) == float(got[r, g])
            assert Fraction(float(got[r, g])) == exact  # exactly representable here


def test_score_associativity_and_duplicate_rows():
    rng = np.random.default_rng(21)
    hb = O.f64_to_bf16(rng.standard_normal((40, 2560)))
    w1 = (0.02 * rng.standard_normal((2560, 256))).astype(np.float32)
    w2 = (0.02 * rng.standard_normal((256, 4))).astype(np.float32)
    s = O.score(hb, w1, w2)
    alt = O.bf16_to_f64(hb) @ (w1.astype(np.float64) @ w2.astype(np.float64))
    np.testing.assert_allclose(s, alt, rtol=2e-6, atol=1e-7)
    hb2 = hb.copy()
    hb2[7] = hb2[31]
    s2 = O.score(hb2, w1, w2)
    assert np.array_equal(s2[7], s2[31])
    # the columns are the four KV groups: permuting W2's columns permutes the scores
    perm = [2, 0, 3, 1]
    np.testing.assert_array_equal(O.score(hb, w1, w2[:, perm]), s[:, perm])


# ---------------------------------------------------------------- commit
def _brute_kept(scores, srcs, cap):
    """Candidate i is kept iff fewer than cap candidates beat it (count-based definition)."""

    def beats(j, i):
        a, b = scores[j], scores[i]
        if np.isnan(a):
            return False if not np.isnan(b) else srcs[j] < srcs[i]
        if np.isnan(b):
            return True
        return a > b or (a == b and srcs[j] < srcs[i])

    n = len(scores)
    return {i for i in range(n) if sum(beats(j, i) for j in range(n) if j != i) < cap}


def _check_slots(keep_idx, n_bank, n_pend, cap, kept_cands):
    # survivors stay, admitted fill free slots ascending in pending order, prefix occupancy
    new_n = min(cap, n_bank + n_pend)
    assert np.all(keep_idx[:new_n] >= 0) and np.all(keep_idx[new_n:] == -1)
    for s in range(n_bank):
        if s in kept_cands:
            assert keep_idx[s] == s
    free = [s for s in range(cap) if not (s < n_bank and s in kept_cands)]
    adm = sorted(i - cap for i in kept_cands if i >= cap)
    for t, s in zip(adm, free):
        assert keep_idx[s] == cap + t


VALUES = [-1.0, -0.0, 0.0, 0.5, 2.0]


@pytest.mark.parametrize("n_bank,n_pend", [(4, 2), (3, 2), (2, 1), (0, 2), (4, 0)])
def test_commit_exhaustive_tiny(n_bank, n_pend):
    cap = 4
    rng = np.random.default_rng(22 + n_bank * 3 + n_pend)
    for vals in itertools.product(VALUES, repeat=n_bank + n_pend):
        srcs = rng.permutation(50)[: n_bank + n_pend]
        bs = np.zeros(cap, np.float32)
        bsrc = np.zeros(cap, np.int32)
        bs[:n_bank] = vals[:n_bank]
        bsrc[:n_bank] = srcs[:n_bank]
        ps = np.array(vals[n_bank:] + (0.0,) * (2 - n_pend), np.float32)
        psrc = np.array(list(srcs[n_bank:]) + [0] * (2 - n_pend), np.int32)
        keep_idx, moves = O.commit_segment(bs, bsrc, n_bank, ps, psrc, n_pend, cap)
        allv = list(vals)
        alls = list(srcs)
        kept = _brute_kept(np.array(allv), alls, cap)
        kept_cands = {i if i < n_bank else cap + (i - n_bank) for i in kept}
        assert {int(k) for k in keep_idx if k >= 0} == kept_cands
        _check_slots(keep_idx, n_bank, n_pend, cap, kept_cands)


def test_commit_nan_ranks_last_and_equal_scores_keep_lowest_src():
    cap = 4
    bs = np.array([np.nan, 1.0, 1.0, 1.0], np.float32)
    bsrc = np.array([0, 9, 3, 7], np.int32)
    ps = np.array([1.0, 1.0], np.float32)
    psrc = np.array([5, 1], np.int32)
    keep_idx, _ = O.commit_segment(bs, bsrc, 4, ps, psrc, 2, cap)
    kept_src = sorted(int(bsrc[k]) if k < cap else int(psrc[k - cap]) for k in keep_idx)
    assert kept_src == [1, 3, 5, 7]
    rng = np.random.default_rng(23)
    st = O.new_layer_state(1, bank=1024, block=256, window=4, head_dim=4)
    st.bank_src[0] = np.stack([rng.permutation(40000)[:1024] for _ in range(4)])
    st.n_bank[0], st.n_pend[0] = 1024, 256
    st.pend_src[0] = np.arange(50000, 50256)
    st.bank_score[...] = 0.25
    st.pend_score[...] = 0.25
    before = st.bank_src.copy()
    O.commit(st)
    for g in range(4):
        lowest = np.sort(np.concatenate([before[0, g], np.arange(50000, 50256)]))[:1024]
        assert np.array_equal(np.sort(st.bank_src[0, g]), lowest)


def test_commit_composability_equals_global_top():
    # after many commits the bank is the best `cap` of every record ever appended
    rng = np.random.default_rng(24)
    cap, block, G = 16, 4, 3
    st = O.new_layer_state(2, window=4, bank=cap, block=block, head_dim=4, groups=G)
    hist = [[[] for _ in range(G)] for _ in range(2)]
    pos = 0
    for _ in range(30):
        npend = rng.integers(1, block + 1)
        for t in range(npend):
            for b in range(2):
                sc = rng.choice([-1.0, 0.0, 0.5, 1.5, float(rng.standard_normal())], size=G)
                st.pend_score[b, t] = sc
                st.pend_src[b, t] = pos
                for g in range(G):
                    hist[b][g].append((O.ordering_key(sc[g], pos), pos))
                    st.pend_k[b, g, t] = pos  # record content = its own position
            pos += 1
        st.n_pend[:] = npend
        O.commit(st)
        for b in range(2):
            for g in range(G):
                best = sorted(hist[b][g])[:cap]
                n = int(st.n_bank[b])
                assert n == len(best)
                assert sorted(st.bank_src[b, g, :n]) == sorted(s for _, s in best)
                assert np.all(st.bank_k[b, g, :n, 0] == st.bank_src[b, g, :n].astype(np.uint16))


def test_commit_order_invariance_and_group_independence():
    rng = np.random.default_rng(25)
    cap = 1024
    bs = rng.standard_normal(cap).astype(np.float32)
    bsrc = rng.permutation(100000)[:cap].astype(np.int32)
    ps = rng.standard_normal(256).astype(np.float32)
    psrc = np.arange(200000, 200256, dtype=np.int32)
    k1, _ = O.commit_segment(bs, bsrc, cap, ps, psrc, 256, cap)
    kept1 = {int(bsrc[k]) if k < cap else int(psrc[k - cap]) for k in k1}
    perm = rng.permutation(cap)
    k2, _ = O.commit_segment(bs[perm], bsrc[perm], cap, ps, psrc, 256, cap)
    kept2 = {int(bsrc[perm][k]) if k < cap else int(psrc[k - cap]) for k in k2}
    assert kept1 == kept2
    # groups select independently; permuting score columns permutes the results
    st = O.new_layer_state(1, bank=64, block=16, window=4, head_dim=4, groups=4)
    st.bank_score[0] = rng.standard_normal((4, 64))
    st.bank_src[0] = np.stack([rng.permutation(1000)[:64] for _ in range(4)])
    st.pend_score[0] = rng.standard_normal((16, 4))
    st.pend_src[0] = np.arange(2000, 2016)
    st.n_bank[0], st.n_pend[0] = 64, 16
    ref = st.copy()
    ka = O.commit(st)
    perm = [3, 1, 0, 2]
    sp = ref.copy()
    sp.bank_score[0] = ref.bank_score[0, perm]
    sp.bank_src[0] = ref.bank_src[0, perm]
    sp.pend_score[0] = ref.pend_score[0][:, perm]
    kb = O.commit(sp)
    np.testing.assert_array_equal(kb[0], ka[0, perm])
    # the same source position may be kept by several groups
    assert len(set(st.bank_src[0, 0]) & set(st.bank_src[0, 1])) > 0
