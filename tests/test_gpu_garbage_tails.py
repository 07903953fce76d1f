"""GPU parity when every slot past the valid counts holds NaN or infinity.

The library documents that only window slots [0, min(pos+1, 1024)), bank slots
[0, n_bank) and pending rows [0, n_pend) are read as records; whatever the rest of
the arrays hold must not reach an output.  A key past the end gets probability 0,
but its value row would still enter the probability x value product, and
0 x NaN is NaN, so the kernels must never take such a row from memory: the
buffer resources the kernels address K/V through cover only the valid rows.
These tests fill every invalid slot (keys, values, FP8 scales, scores, sources)
with NaN and infinity patterns, at counts that leave partial tiles, and require
the oracle's results (which only ever look at valid slots) and finite
log-sum-exps.  Every access stays inside the allocated arrays.
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import fp8_ref as F
from oracle import int8_ref as I
import swa_memory_anchor_amd as R
import synth
from synth import core as C

from gpu_util import (DEV, KV, assert_attn_close, assert_keys_close, bf16_dev, bits_host,
                      decode_gpu, decode_gpu_fp8, decode_gpu_i8, download, download_fp8, f32_dev,
                      norm_dev, upload, upload_fp8)

pytestmark = pytest.mark.gpu

BF16_BAD = np.array([0x7FC0, 0x7F80, 0xFF80, 0xFFFF, 0x7FFF], np.uint16)  # NaN, +-inf, NaNs
E4M3_BAD = np.array([0x7F, 0xFF], np.uint8)  # the two E4M3 NaN codes
I8_BAD = np.array([0x80, 0x7F, 0x81], np.uint8)  # -128 (never written), +127, -127
F32_BAD = np.array([np.nan, np.inf, -np.inf], np.float32)

# (n_bank, n_pend, pos): partial 16- and 32-key tiles in every segment, empty
# segments, a window that has not wrapped yet
COUNTS = [(37, 5, 600), (513, 129, 100), (0, 1, 0), (1, 0, 16), (1023, 255, 1021),
          (16, 16, 15), (0, 0, -1), (700, 200, 5)]


def _bad_fill(shape, pattern):
    return np.resize(pattern, int(np.prod(shape))).reshape(shape)


def _valid_masks(st):
    """Boolean masks over the slot axis of window, bank and pending, per sequence."""
    B = st.pos.shape[0]
    win = np.zeros((B, O.WINDOW), bool)
    bank = np.zeros((B, O.BANK), bool)
    pend = np.zeros((B, O.BLOCK), bool)
    for b in range(B):
        win[b, :min(int(st.pos[b]) + 1, O.WINDOW)] = True
        bank[b, :int(st.n_bank[b])] = True
        pend[b, :int(st.n_pend[b])] = True
    return win, bank, pend


def _poison_bf16(st):
    """Overwrite every invalid slot of a BF16 oracle state with NaN/inf patterns."""
    win, bank, pend = _valid_masks(st)
    for nm, m in (("win_k", win), ("win_v", win), ("bank_k", bank), ("bank_v", bank),
                  ("pend_k", pend), ("pend_v", pend)):
        a = getattr(st, nm)
        bad = _bad_fill(a.shape, BF16_BAD)
        inv = ~m[:, None, :, None]
        a[...] = np.where(inv, bad, a)
    st.bank_score[...] = np.where(bank[:, None, :], st.bank_score,
                                  _bad_fill(st.bank_score.shape, F32_BAD))
    st.pend_score[...] = np.where(pend[:, :, None], st.pend_score,
                                  _bad_fill(st.pend_score.shape, F32_BAD))
    return st


def _state(tag, counts):
    B = len(counts)
    st = O.new_layer_state(B)
    for nm in KV:
        a = getattr(st, nm)
        a[...] = synth.normal_bf16_np(synth.stream_key(tag, nm), a.size).reshape(a.shape)
    st.bank_score[...] = synth.normal_f32_np(synth.stream_key(tag, "bs"), st.bank_score.shape)
    st.pend_score[...] = synth.normal_f32_np(synth.stream_key(tag, "ps"), st.pend_score.shape)
    for b, (nb, npd, pos) in enumerate(counts):
        st.n_bank[b], st.n_pend[b], st.pos[b] = nb, npd, pos
        for g in range(4):
            st.bank_src[b, g] = synth.distinct_ints_np(synth.stream_key(tag, "src", b, g), 1024,
                                                       10**6, 10**6 + 4096)
        st.pend_src[b] = np.arange(256) + 2 * 10**6
    return _poison_bf16(st)


def _gains(tag):
    return {nm: synth.normal_f32_np(synth.stream_key(tag, nm), (256,), 1.0, 0.1)
            for nm in ("gq_win", "gk_win", "gq_rma", "gk_rma")}


def _check_outputs(outs, ref, what):
    o_w, l_w, o_r, l_r = outs
    for x in (l_w, l_r):
        v = x.cpu().numpy()
        assert not np.any(np.isnan(v)), what
    assert_attn_close(bits_host(o_w), l_w.cpu().numpy(), ref[0], ref[1], what=f"{what} window")
    assert_attn_close(bits_host(o_r), l_r.cpu().numpy(), ref[2], ref[3], what=f"{what} anchor")


@pytest.mark.parametrize("batch_rep", [1, 8])
def test_decode_ignores_poisoned_tails(batch_rep):
    # batch 8 splits every branch; batch 64 does not
    counts = COUNTS * batch_rep
    B = len(counts)
    print(f"case: poisoned decode B={B} splits={R.rma_decode_splits(B)}", flush=True)
    st = _state("poison_dec", counts)
    g = _gains("poison_dec")
    q = synth.normal_bf16_np(synth.stream_key("poison_dec", "q"), B * 4096).reshape(B, 16, 256)
    qd = bf16_dev(q)
    outs = decode_gpu(upload(st), qd, qd, norm_dev(g))
    torch.cuda.synchronize()
    ref = O.decode(st, q, q, g["gq_win"], g["gq_rma"], 1e-6, 1e7)
    _check_outputs(outs, ref, f"poisoned decode B={B}")


def test_fused_step_ignores_poisoned_tails():
    print("case: poisoned fused step", flush=True)
    B = len(COUNTS)
    st = _state("poison_step", COUNTS)
    g = _gains("poison_step")
    recs = [synth.normal_bf16_np(synth.stream_key("poison_step", "rec", i), B * 1024).reshape(
        B, 4, 256) for i in range(4)]
    q = synth.normal_bf16_np(synth.stream_key("poison_step", "q"), B * 4096).reshape(B, 16, 256)
    dst = upload(st)
    qd = bf16_dev(q)
    outs = [torch.empty(B, 16, 256, dtype=torch.bfloat16, device=DEV),
            torch.empty(B, 16, device=DEV),
            torch.empty(B, 16, 256, dtype=torch.bfloat16, device=DEV),
            torch.empty(B, 16, device=DEV)]
    R.swa_rma_step(dst, B, *[bf16_dev(r) for r in recs], None, qd, qd, norm_dev(g), *outs,
                   R.step_workspace(B))
    torch.cuda.synchronize()
    O.append(st, *recs, g["gk_win"], g["gk_rma"], 1e-6, 1e7)
    ref = O.decode(st, q, q, g["gq_win"], g["gq_rma"], 1e-6, 1e7)
    _check_outputs(outs, ref, "poisoned step")
    got = download(dst)
    for k in ("n_pend", "pos", "pend_src"):
        assert np.array_equal(getattr(got, k), getattr(st, k)), k
    for k in ("win_k", "pend_k"):
        assert_keys_close(getattr(got, k), getattr(st, k), what=f"poisoned step {k}")


def test_prefill_ignores_poisoned_tails():
    C_ = 40
    counts = [(37, 5, 600), (0, 0, -1), (513, 100, 100), (1024, 56, 70000), (5, 0, 3)]
    B = len(counts)
    print(f"case: poisoned prefill B={B} C={C_}", flush=True)
    st = _state("poison_pf", counts)
    g = _gains("poison_pf")
    recs = [synth.normal_bf16_np(synth.stream_key("poison_pf", "rec", i), B * C_ * 1024).reshape(
        B, C_, 4, 256) for i in range(4)]
    q = synth.normal_bf16_np(synth.stream_key("poison_pf", "q"), B * C_ * 4096).reshape(
        B, C_, 16, 256)
    dst = upload(st)
    qd = bf16_dev(q)
    o_w = torch.empty(B, C_, 16, 256, dtype=torch.bfloat16, device=DEV)
    o_r = torch.empty_like(o_w)
    l_w = torch.empty(B, C_, 16, device=DEV)
    l_r = torch.empty_like(l_w)
    R.swa_rma_prefill(dst, B, C_, *[bf16_dev(r) for r in recs], None, qd, qd, norm_dev(g),
                      o_w, l_w, o_r, l_r, R.prefill_workspace(B, C_))
    torch.cuda.synchronize()
    ow, lw, orr, lr = bits_host(o_w), l_w.cpu().numpy(), bits_host(o_r), l_r.cpu().numpy()
    assert not np.any(np.isnan(lw)) and not np.any(np.isnan(lr))
    for b in range(B):
        one = O.new_layer_state(1)
        for k in one.__dict__:
            getattr(one, k)[...] = getattr(st, k)[b:b + 1]
        refs = []
        for i in range(C_):
            O.append(one, *[r[b:b + 1, i] for r in recs], g["gk_win"], g["gk_rma"], 1e-6, 1e7)
            refs.append(O.decode(one, q[b:b + 1, i], q[b:b + 1, i], g["gq_win"], g["gq_rma"],
                                 1e-6, 1e7))
        assert_attn_close(ow[b], lw[b], np.stack([d[0][0] for d in refs]),
                          np.stack([d[1][0] for d in refs]), what=f"poisoned prefill b={b} win")
        assert_attn_close(orr[b], lr[b], np.stack([d[2][0] for d in refs]),
                          np.stack([d[3][0] for d in refs]), what=f"poisoned prefill b={b} rma")


def test_commit_ignores_poisoned_tails():
    print("case: poisoned commit", flush=True)
    B = len(COUNTS)
    st = _state("poison_commit", COUNTS)
    dst = upload(st)
    keep = torch.empty(B, 4, 1024, dtype=torch.int32, device=DEV)
    R.rma_commit_topk(dst, B, keep)
    torch.cuda.synchronize()
    ref = st.copy()
    k_ref = O.commit(ref)
    assert np.array_equal(keep.cpu().numpy(), k_ref)
    got = download(dst)
    for b in range(B):
        n = int(ref.n_bank[b])
        for k in ("bank_k", "bank_v", "bank_score", "bank_src"):
            a, r = getattr(got, k)[b, :, :n], getattr(ref, k)[b, :, :n]
            if a.dtype == np.float32:
                a, r = a.view(np.uint32), r.view(np.uint32)
            assert np.array_equal(a, r), (b, k)
    assert np.array_equal(got.n_bank, ref.n_bank) and np.all(got.n_pend == 0)


def _fp8_state(tag, counts):
    st = F.new_layer_state_fp8(len(counts))
    for nm in KV:
        a = getattr(st, nm)
        a[...] = C.normal_e4m3_np(synth.stream_key(tag, nm), a.size).reshape(a.shape)
        s = getattr(st, nm + "s")
        s[...] = C.row_scale_np(synth.stream_key(tag, nm, "s"), s.size).reshape(s.shape)
    for b, (nb, npd, pos) in enumerate(counts):
        st.n_bank[b], st.n_pend[b], st.pos[b] = nb, npd, pos
    win, bank, pend = _valid_masks(st)
    for nm, m in (("win_k", win), ("win_v", win), ("bank_k", bank), ("bank_v", bank),
                  ("pend_k", pend), ("pend_v", pend)):
        a = getattr(st, nm)
        a[...] = np.where(~m[:, None, :, None], _bad_fill(a.shape, E4M3_BAD), a)
        s = getattr(st, nm + "s")
        s[...] = np.where(~m[:, None, :], _bad_fill(s.shape, F32_BAD), s)
    return st


@pytest.mark.parametrize("batch_rep", [1, 8])
def test_fp8_decode_ignores_poisoned_tails(batch_rep):
    counts = COUNTS * batch_rep
    B = len(counts)
    print(f"case: poisoned fp8 decode B={B}", flush=True)
    st = _fp8_state("poison_fp8", counts)
    g = _gains("poison_fp8")
    q = synth.normal_bf16_np(synth.stream_key("poison_fp8", "q"), B * 4096).reshape(B, 16, 256)
    qd = bf16_dev(q)
    outs = decode_gpu_fp8(upload_fp8(st), qd, qd, norm_dev(g))
    torch.cuda.synchronize()
    ref = F.decode(st, q, q, g["gq_win"], g["gq_rma"], 1e-6, 1e7)
    _check_outputs(outs, ref, f"poisoned fp8 decode B={B}")
    # the FP8 commit moves scales with rows and reads nothing past the counts either
    dst = upload_fp8(st)
    keep = torch.empty(B, 4, 1024, dtype=torch.int32, device=DEV)
    st.bank_score[...] = synth.normal_f32_np(synth.stream_key("poison_fp8", "bs"),
                                             st.bank_score.shape)
    st.pend_score[...] = synth.normal_f32_np(synth.stream_key("poison_fp8", "ps"),
                                             st.pend_score.shape)
    for b in range(B):
        for gg in range(4):
            st.bank_src[b, gg] = synth.distinct_ints_np(
                synth.stream_key("poison_fp8", "src", b, gg), 1024, 10**6, 10**6 + 4096)
        st.pend_src[b] = np.arange(256) + 2 * 10**6
    dst = upload_fp8(st)
    R.rma_commit_topk_fp8(dst, B, keep)
    torch.cuda.synchronize()
    ref_st = st.copy()
    k_ref = F.commit(ref_st)
    assert np.array_equal(keep.cpu().numpy(), k_ref)
    got = download_fp8(dst)
    for b in range(B):
        n = int(ref_st.n_bank[b])
        for k in ("bank_k", "bank_v", "bank_ks", "bank_vs", "bank_src"):
            a, r = getattr(got, k)[b, :, :n], getattr(ref_st, k)[b, :, :n]
            if a.dtype == np.float32:
                a, r = a.view(np.uint32), r.view(np.uint32)
            assert np.array_equal(a, r), (b, k)


def _i8_state(tag, counts):
    """INT8 state whose invalid slots hold extreme codes (-128 included, which the
    quantiser never writes) and NaN/infinite row scales, so any such row that took part
    in a dot product or the probability x value sum would make the output non-finite."""
    st = I.new_layer_state_i8(len(counts))
    for nm in KV:
        a = getattr(st, nm)
        a[...] = C.normal_i8_np(synth.stream_key(tag, nm), a.size).reshape(a.shape)
        s = getattr(st, nm + "s")
        s[...] = C.row_scale_np(synth.stream_key(tag, nm, "s"), s.size, denom=128).reshape(s.shape)
    for b, (nb, npd, pos) in enumerate(counts):
        st.n_bank[b], st.n_pend[b], st.pos[b] = nb, npd, pos
    win, bank, pend = _valid_masks(st)
    for nm, m in (("win_k", win), ("win_v", win), ("bank_k", bank), ("bank_v", bank),
                  ("pend_k", pend), ("pend_v", pend)):
        a = getattr(st, nm)
        a[...] = np.where(~m[:, None, :, None], _bad_fill(a.shape, I8_BAD), a)
        s = getattr(st, nm + "s")
        s[...] = np.where(~m[:, None, :], _bad_fill(s.shape, F32_BAD), s)
    return st


@pytest.mark.parametrize("batch_rep", [1, 8])
def test_int8_decode_ignores_poisoned_tails(batch_rep):
    counts = COUNTS * batch_rep
    B = len(counts)
    print(f"case: poisoned int8 decode B={B}", flush=True)
    st = _i8_state("poison_i8", counts)
    g = _gains("poison_i8")
    q = synth.normal_bf16_np(synth.stream_key("poison_i8", "q"), B * 4096).reshape(B, 16, 256)
    qd = bf16_dev(q)
    outs = decode_gpu_i8(upload_fp8(st), qd, qd, norm_dev(g))
    torch.cuda.synchronize()
    ref = I.decode(st, q, q, g["gq_win"], g["gq_rma"], 1e-6, 1e7)
    _check_outputs(outs, ref, f"poisoned int8 decode B={B}")
