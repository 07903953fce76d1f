"""Pins of the oracle's softmax attention and of the decode step's branch wiring."""

import math

import numpy as np
import torch

import oracle as O


def _sdpa(q, k, v):
    qt, kt, vt = (torch.from_numpy(a)[None, None] for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0].numpy()
    lse = torch.logsumexp(torch.from_numpy(q @ k.T) / math.sqrt(q.shape[1]), dim=1).numpy()
    return o, lse


def test_attend_matches_torch_sdpa_float64():
    rng = np.random.default_rng(10)
    for n in (1, 7, 1024, 1280):
        q = rng.standard_normal((4, 256)) * 2
        k = rng.standard_normal((n, 256))
        v = rng.standard_normal((n, 256))
        o, lse = O.attend(q, k, v)
        ro, rl = _sdpa(q, k, v)
        np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, rl, rtol=1e-13)


def test_attend_special_cases():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((4, 256))
    k1 = rng.standard_normal((1, 256))
    v1 = rng.standard_normal((1, 256))
    o, lse = O.attend(q, k1, v1)
    np.testing.assert_allclose(o, np.repeat(v1, 4, 0), rtol=1e-15)
    np.testing.assert_allclose(lse, (q @ k1[0]) / 16.0, rtol=1e-14)
    # N identical keys: the mean of the values, lse = s + ln N
    kN = np.repeat(k1, 37, 0)
    vN = rng.standard_normal((37, 256))
    o, lse = O.attend(q, kN, vN)
    np.testing.assert_allclose(o, np.repeat(vN.mean(0, keepdims=True), 4, 0), rtol=1e-12,
                               atol=1e-14)
    np.testing.assert_allclose(lse, (q @ k1[0]) / 16.0 + math.log(37), rtol=1e-13)
    # zero query: uniform weights, lse = ln N
    o, lse = O.attend(np.zeros((4, 256)), rng.standard_normal((50, 256)), vN[:1].repeat(50, 0))
    np.testing.assert_allclose(lse, math.log(50), rtol=1e-15)
    # no keys at all
    o, lse = O.attend(q, np.zeros((0, 256)), np.zeros((0, 256)))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_lse_merge_identity_and_permutation_invariance():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((4, 256))
    k = rng.standard_normal((300, 256))
    v = rng.standard_normal((300, 256))
    o, lse = O.attend(q, k, v)
    o1, l1 = O.attend(q, k[:123], v[:123])
    o2, l2 = O.attend(q, k[123:], v[123:])
    om, lm = O.merge_lse(o1, l1, o2, l2)
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lm, lse, rtol=1e-14)
    perm = rng.permutation(300)
    op, lp = O.attend(q, k[perm], v[perm])
    np.testing.assert_allclose(op, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lp, lse, rtol=1e-14)


def _state_with(rng, n_bank, n_pend, pos):
    st = O.new_layer_state(1)
    for nm in ("win_k", "win_v", "bank_k", "bank_v", "pend_k", "pend_v"):
        arr = getattr(st, nm)
        arr[...] = O.f64_to_bf16(rng.standard_normal(arr.shape))
    st.n_bank[0], st.n_pend[0], st.pos[0] = n_bank, n_pend, pos
    return st


def test_decode_head_to_group_mapping_and_branch_contents():
    rng = np.random.default_rng(13)
    st = _state_with(rng, 1024, 256, 5000)
    # values of group g are the constant g + 1 in both branches
    for g in range(4):
        for nm in ("win_v", "bank_v", "pend_v"):
            getattr(st, nm)[0, g] = O.f64_to_bf16(g + 1.0)
    q = O.f64_to_bf16(rng.standard_normal((1, 16, 256)))
    ones = np.ones(256)
    ow, lw, orr, lr = O.decode(st, q, q, ones, ones, 1e-6, 1e7)
    for h in range(16):
        np.testing.assert_allclose(ow[0, h], h // 4 + 1.0, rtol=1e-14)
        np.testing.assert_allclose(orr[0, h], h // 4 + 1.0, rtol=1e-14)


def test_decode_reads_only_valid_slots():
    rng = np.random.default_rng(14)
    st = _state_with(rng, 3, 2, 9)  # window holds positions 0..9 in slots 0..9
    q = O.f64_to_bf16(rng.standard_normal((1, 16, 256)))
    ones = np.ones(256)
    ref = O.decode(st, q, q, ones, ones, 1e-6, 1e7)
    poisoned = st.copy()
    poisoned.win_v[:, :, 10:] = O.f64_to_bf16(1e30)
    poisoned.bank_v[:, :, 3:] = O.f64_to_bf16(1e30)
    poisoned.pend_v[:, :, 2:] = O.f64_to_bf16(1e30)
    got = O.decode(poisoned, q, q, ones, ones, 1e-6, 1e7)
    for a, b in zip(ref, got):
        np.testing.assert_array_equal(a, b)
    # the anchor branch is one softmax over bank then pending
    qh = O.rope(O.rms_norm(O.bf16_to_f64(q[0, 5]), ones, 1e-6), 9, 1e7)
    keys = np.concatenate([st.bank_k[0, 1, :3], st.pend_k[0, 1, :2]])
    vals = np.concatenate([st.bank_v[0, 1, :3], st.pend_v[0, 1, :2]])
    o, l = O.attend(qh[None], O.bf16_to_f64(keys), O.bf16_to_f64(vals))
    np.testing.assert_allclose(ref[2][0, 5], o[0], rtol=1e-13)
    np.testing.assert_allclose(ref[3][0, 5], l[0], rtol=1e-14)
    # the window branch reads exactly the ten slots holding positions 0..9
    o, l = O.attend(qh[None], O.bf16_to_f64(st.win_k[0, 1, :10]), O.bf16_to_f64(st.win_v[0, 1, :10]))
    np.testing.assert_allclose(ref[0][0, 5], o[0], rtol=1e-13)
    np.testing.assert_allclose(ref[1][0, 5], l[0], rtol=1e-14)
    # once the ring has wrapped, all 1024 slots are read
    st.pos[0] = 5000
    full = O.decode(st, q, q, ones, ones, 1e-6, 1e7)
    qh = O.rope(O.rms_norm(O.bf16_to_f64(q[0, 5]), ones, 1e-6), 5000, 1e7)
    o, l = O.attend(qh[None], O.bf16_to_f64(st.win_k[0, 1]), O.bf16_to_f64(st.win_v[0, 1]))
    np.testing.assert_allclose(full[0][0, 5], o[0], rtol=1e-13)


def test_decode_rotates_query_at_current_position():
    # a single key written at position s and read at position p depends only on p - s
    rng = np.random.default_rng(15)
    ones = np.ones(256)
    q = O.f64_to_bf16(rng.standard_normal((1, 16, 256)))
    kraw = rng.standard_normal(256)
    lses = []
    for p in (40, 40 + 4096):
        st = O.new_layer_state(1)
        st.win_k[0, :, p % 1024] = O.f64_to_bf16(O.rope(kraw, p, 1e7))
        st.pos[0] = p
        # only one valid window slot: pretend the stream started at p
        kk = st.win_k[0, :, p % 1024:p % 1024 + 1]
        o, l = O.decode_one([kk[g] for g in range(4)], [np.zeros((1, 256), np.uint16)] * 4,
                            q[0], ones, p, 1e-6, 1e7)
        lses.append(l)
    np.testing.assert_allclose(lses[0], lses[1], atol=1e-2)  # BF16 rounding of the key
