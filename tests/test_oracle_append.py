"""Pins of the oracle's append (the write of one token into window and pending block).

What is pinned, from the pages about EdgeRock-4B:
  * fluxbbs.com, "EdgeRock-4B 开源：72 MiB 固定 KV，AIME 82.9 分", section
    "架构：递归、局部窗口与记忆锚点三件套": keys carry a learned RMS norm and partial
    rotary (64 of 256 dims, base 1e7); values are neither normalised nor rotated;
    the window branch and the anchor branch are separate modules with their own
    parameters.
  * section "72 MiB 是怎么算出来的": a 1024-position window per group, a 256-record
    pending block, BF16 records.
  * neodrop.ai, "内存还会跌吗？KV Cache砍掉99%…", section "三段记忆，只记值得记的":
    one candidate record per generated token.

The expected rows are built here from library routines, not from the oracle's own
formulas: torch's RMS norm and the rotary embedding of the transformers Llama code
(rotate-half pairing, frequencies in float32).  The slot, counter and source
conventions are checked against positions the test derives from its own inputs.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synth

EPS, BASE = 1e-6, 1e7


def _rotary_ref(x, pos):
    """Rows x [n][256] float64, rotated at integer positions pos [n] by the
    transformers Llama rotary code on dims 0..63 (dims 64.. pass through)."""
    from transformers import LlamaConfig
    from transformers.models.llama import modeling_llama as m

    cfg = LlamaConfig(hidden_size=256, num_attention_heads=4, head_dim=64, rope_theta=BASE,
                      max_position_embeddings=262144)
    emb = m.LlamaRotaryEmbedding(cfg)
    xt = torch.from_numpy(np.ascontiguousarray(x[None, None, :, :64]))
    cos, sin = emb(xt, torch.tensor([list(pos)]))
    rot, _ = m.apply_rotary_pos_emb(xt, xt, cos, sin)
    y = x.copy()
    y[:, :64] = rot[0, 0].numpy()
    return y


def _norm_ref(x_bits, gamma):
    x = torch.from_numpy(O.bf16_to_f64(x_bits))
    return torch.nn.functional.rms_norm(x, (256,), torch.from_numpy(gamma), eps=EPS).numpy()


def _assert_bf16_near(stored_bits, ref, pos, what):
    """Stored BF16 rows within one BF16 ulp of the float64 reference, plus the
    float32-frequency error of the library rotary (angle error <= pos * 2^-23)."""
    got = O.bf16_to_f64(stored_bits)
    _, e = np.frexp(ref)
    ulp = np.ldexp(1.0, e - 8)
    row = np.abs(ref).max(axis=-1, keepdims=True)
    slack = (np.asarray(pos, np.float64)[:, None] + 1.0) * 2.0**-21 * row
    err = np.abs(got - ref)
    assert np.all(err <= ulp + slack), (what, float((err / (ulp + slack)).max()))


def _state(counts, seed):
    """A state with every array filled with random bits, then the given counters."""
    B = len(counts)
    st = O.new_layer_state(B)
    rng = np.random.default_rng(seed)
    for nm in ("win_k", "win_v", "bank_k", "bank_v", "pend_k", "pend_v"):
        a = getattr(st, nm)
        a[...] = O.f64_to_bf16(rng.standard_normal(a.shape))
    st.bank_score[...] = rng.standard_normal(st.bank_score.shape)
    st.pend_score[...] = rng.standard_normal(st.pend_score.shape)
    st.bank_src[...] = rng.integers(0, 1 << 20, st.bank_src.shape)
    st.pend_src[...] = rng.integers(0, 1 << 20, st.pend_src.shape)
    for b, (nb, npd, pos) in enumerate(counts):
        st.n_bank[b], st.n_pend[b], st.pos[b] = nb, npd, pos
    return st


# (n_bank, n_pend, pos): a fresh stream, the last slot before the ring wraps, the
# wrap itself, a wrapped ring, and the append that fills the pending block.
COUNTS = [(0, 0, -1), (17, 3, 1022), (1024, 40, 1023), (300, 128, 1500), (1024, 255, 1279)]


def test_append_writes_the_defined_rows_and_nothing_else():
    st = _state(COUNTS, 11)
    before = st.copy()
    B = len(COUNTS)
    rng = np.random.default_rng(12)
    k_win, v_win, k_rma, v_rma = (O.f64_to_bf16(rng.standard_normal((B, 4, 256)))
                                  for _ in range(4))
    gk_win = 1.0 + 0.1 * rng.standard_normal(256)
    gk_rma = 1.0 + 0.1 * rng.standard_normal(256)
    score = rng.standard_normal((B, 4)).astype(np.float32)
    O.append(st, k_win, v_win, k_rma, v_rma, gk_win, gk_rma, EPS, BASE, score=score)

    for b, (nb, npd, pos) in enumerate(COUNTS):
        p = pos + 1  # the new token's position
        slot = [0, 1023, 0, 477, 256][b]  # p mod 1024, written out per case
        assert slot == p % 1024
        t = npd
        # window key: the window gain, rotated at the new position
        ref_w = _rotary_ref(_norm_ref(k_win[b], gk_win), [p] * 4)
        _assert_bf16_near(st.win_k[b, :, slot], ref_w, [p] * 4, f"win_k b={b}")
        # candidate key: the anchor gain, same position
        ref_r = _rotary_ref(_norm_ref(k_rma[b], gk_rma), [p] * 4)
        _assert_bf16_near(st.pend_k[b, :, t], ref_r, [p] * 4, f"pend_k b={b}")
        # values stored raw, bit for bit
        assert np.array_equal(st.win_v[b, :, slot], v_win[b])
        assert np.array_equal(st.pend_v[b, :, t], v_rma[b])
        assert st.pend_src[b, t] == p
        assert np.array_equal(st.pend_score[b, t], score[b])
        assert st.n_pend[b] == npd + 1 and st.pos[b] == p and st.n_bank[b] == nb
        # every other slot and row is untouched
        for nm, idx in (("win_k", slot), ("win_v", slot), ("pend_k", t), ("pend_v", t)):
            a, a0 = getattr(st, nm)[b], getattr(before, nm)[b]
            keep = np.ones(a.shape[1], bool)
            keep[idx] = False
            assert np.array_equal(a[:, keep], a0[:, keep]), (nm, b)
        keep = np.ones(256, bool)
        keep[t] = False
        assert np.array_equal(st.pend_src[b, keep], before.pend_src[b, keep])
        assert np.array_equal(st.pend_score[b, keep], before.pend_score[b, keep])
    for nm in ("bank_k", "bank_v", "bank_score", "bank_src"):
        assert np.array_equal(getattr(st, nm), getattr(before, nm)), nm


def test_append_without_score_leaves_the_score_row():
    st = _state([(5, 9, 100)], 13)
    before = st.copy()
    rng = np.random.default_rng(14)
    rec = [O.f64_to_bf16(rng.standard_normal((1, 4, 256))) for _ in range(4)]
    O.append(st, *rec, np.ones(256), np.ones(256), EPS, BASE)
    assert np.array_equal(st.pend_score, before.pend_score)
    assert st.pend_src[0, 9] == 101 and st.n_pend[0] == 10


def test_append_refuses_a_full_pending_block():
    st = _state([(1024, 256, 5000)], 15)
    rec = [np.zeros((1, 4, 256), np.uint16) for _ in range(4)]
    with pytest.raises(AssertionError):
        O.append(st, *rec, np.ones(256), np.ones(256), EPS, BASE)


def test_window_after_1500_appends_holds_the_last_1024_positions():
    """Stream 1500 tokens (committing whenever the pending block fills).  Each value
    row carries its own position in two exactly representable BF16 elements, so the
    ring's contents can be read back: slot s must hold the position p in 476..1499
    with p mod 1024 = s; the keys there must be the keys of that position."""
    n = 1500
    st = O.new_layer_state(1)
    g1 = np.ones(256)
    rng = synth.rng_np(synth.stream_key("append_pin", "scores"))
    k_rows = O.f64_to_bf16(np.random.default_rng(16).standard_normal((n, 4, 256)))
    for p in range(n):
        if st.n_pend[0] == st.block:
            st.pend_score[...] = rng.standard_normal(st.pend_score.shape)
            O.commit(st)
        v = np.zeros((1, 4, 256))
        v[..., 0], v[..., 1] = p // 64, p % 64
        vb = O.f64_to_bf16(v)
        O.append(st, k_rows[p][None], vb, k_rows[p][None], vb, g1, g1, EPS, BASE)
    assert st.pos[0] == n - 1
    stored = O.bf16_to_f64(st.win_v[0, :, :, :2])  # [4][1024][2]
    held = stored[..., 0] * 64 + stored[..., 1]
    expect = np.array([s + 1024 if s + 1024 < n else s for s in range(1024)], np.float64)
    assert np.all(expect >= n - 1024)
    assert np.array_equal(held, np.broadcast_to(expect, held.shape))
    # pending rows since the last commit (1280 = 5 * 256 committed): 1280..1499
    assert st.n_pend[0] == n - 1280
    assert np.array_equal(st.pend_src[0, :n - 1280], np.arange(1280, n))
    pv = O.bf16_to_f64(st.pend_v[0, :, :n - 1280, :2])
    assert np.array_equal(pv[..., 0] * 64 + pv[..., 1],
                          np.broadcast_to(np.arange(1280, n), (4, n - 1280)))
    # window keys: slot s holds the key of the position it holds, rotated there
    for s in (0, 475, 476, 1023):
        p = int(expect[s])
        ref = _rotary_ref(_norm_ref(k_rows[p], g1), [p] * 4)
        _assert_bf16_near(st.win_k[0, :, s], ref, [p] * 4, f"slot {s}")
