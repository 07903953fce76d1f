"""GPU parity on the batch-1 long stream: 262144 positions through all 8 layers.

Per token and layer the stream runs one fused step (swa_rma_step: append to
window + pending, then decode, as the benchmark's stream does); every 256 tokens
each layer commits.  Candidate scores come from the input generator (passed
through the step), so the commit chain of the GPU and of the
oracle see identical scores and must agree bit for bit; the scorer itself is
checked separately on sampled blocks of the stream's hidden states.

Checked against the oracle:
* keep_idx of all 1024 commits of layers 0 and 7 (oracle chain, one selection
  per group and commit);
* the final bank of every layer holds exactly the global best 1024 of all
  262144 records of each group (composability of the per-block commits);
* decode outputs at sampled positions (ring not yet full, block boundaries,
  deep in the stream, the last position) in layers 0 and 7, with the state
  rebuilt by the oracle from the seeds: window = the last 1024 positions, bank
  = its own chain, pending = the current block;
* the state's size never changes.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import swa_memory_anchor_amd as R
from synth import workloads as W

from gpu_util import (DEV, assert_attn_close, assert_scores_close, bf16_dev, bits_host, f32_dev,
                      norm_dev)

pytestmark = pytest.mark.gpu

WL = W.LONG_STREAM_B1
T = WL.position
NBLK = T // O.BLOCK
CHUNK = 4096  # tokens generated on the device at a time
CHECK_LAYERS = (0, 7)
SAMPLES = (0, 1, 2, 255, 256, 257, 1023, 1024, 1025, 1279, 1280, 2047, 4095, 4096, 65535, 65536,
           131071, 200003, 262143)


def _oracle_keys(layer, name, gain, positions):
    """Stored keys for records at `positions` (BF16 bits [n][4][256]), as the oracle writes them."""
    raw = O.bf16_to_f64(W.record_rows_np(WL, layer, name, positions))
    out = np.empty(raw.shape, np.uint16)
    for i, p in enumerate(positions):
        out[i] = O.f64_to_bf16(O.rope(O.rms_norm(raw[i], gain, WL.eps), int(p), WL.rope_base))
    return out


def _oracle_chain(layer, snap_blocks):
    """The oracle's commit chain (scores and sources only) over all blocks of a layer.

    Returns keep_idx [NBLK][4][1024] and bank_src snapshots after the commits
    numbered in snap_blocks (the state a decode in block c+1 sees)."""
    bs = np.zeros((4, O.BANK), np.float32)
    bsrc = np.zeros((4, O.BANK), np.int32)
    nb = 0
    keeps = np.empty((NBLK, 4, O.BANK), np.int32)
    snaps = {}
    for c in range(NBLK):
        ps = W.stream_scores_np(WL, layer, c)
        psrc = np.arange(c * O.BLOCK, (c + 1) * O.BLOCK, dtype=np.int32)
        for g in range(4):
            ki, moves = O.commit_segment(bs[g], bsrc[g], nb, ps[:, g], psrc, O.BLOCK, O.BANK)
            keeps[c, g] = ki
            for t, s in moves:
                bs[g, s] = ps[t, g]
                bsrc[g, s] = psrc[t]
        nb = min(O.BANK, nb + O.BLOCK)
        if c in snap_blocks:
            snaps[c] = (bsrc.copy(), nb)
    return keeps, snaps


def test_long_stream_b1():
    L = WL.layers
    lib = R.lib()
    stream = torch.cuda.current_stream().cuda_stream
    states = [R.alloc_layer_state(1) for _ in range(L)]
    gains = [W.gains(WL, l) for l in range(L)]
    norms = [norm_dev(g, WL.eps, WL.rope_base) for g in gains]
    st_c = [ctypes.byref(R._state_c(s)) for s in states]
    nm_c = [ctypes.byref(R._norm_c(n)) for n in norms]
    state_bytes = sum(t.numel() * t.element_size() for t in states[0].__dict__.values())
    assert state_bytes == R.rma_layer_state_bytes(1)

    rec = {nm: torch.empty(L, CHUNK, 4, 256, dtype=torch.bfloat16, device=DEV)
           for nm in W.RECORD_NAMES}
    qb = torch.empty(L, CHUNK, 16, 256, dtype=torch.bfloat16, device=DEV)
    sb = torch.empty(L, CHUNK, 4, dtype=torch.float32, device=DEV)
    outs = [(torch.empty(1, 16, 256, dtype=torch.bfloat16, device=DEV),
             torch.empty(1, 16, dtype=torch.float32, device=DEV),
             torch.empty(1, 16, 256, dtype=torch.bfloat16, device=DEV),
             torch.empty(1, 16, dtype=torch.float32, device=DEV)) for _ in range(L)]
    out_p = [[o.data_ptr() for o in os_] for os_ in outs]
    ws = R.step_workspace(1)
    ws_p, ws_n = ws.data_ptr(), ws.numel()
    keeps = torch.empty(NBLK, L, 4, O.BANK, dtype=torch.int32, device=DEV)
    captured = {}
    samples = set(SAMPLES)
    rec_stride = 4 * 256 * 2
    q_stride = 16 * 256 * 2
    for c0 in range(0, T, CHUNK):
        for l in range(L):
            for nm in W.RECORD_NAMES:
                W.record_torch_(WL, l, nm, c0, rec[nm][l])
            W.stream_q_torch_(WL, l, c0, qb[l])
            sc = np.concatenate([W.stream_scores_np(WL, l, c) for c in
                                 range(c0 // O.BLOCK, (c0 + CHUNK) // O.BLOCK)])
            sb[l].copy_(torch.from_numpy(sc))
        base = {nm: [rec[nm][l].data_ptr() for l in range(L)] for nm in W.RECORD_NAMES}
        qbase = [qb[l].data_ptr() for l in range(L)]
        sbase = [sb[l].data_ptr() for l in range(L)]
        for t in range(CHUNK):
            p = c0 + t
            for l in range(L):
                r = [base[nm][l] + t * rec_stride for nm in W.RECORD_NAMES]
                q = qbase[l] + t * q_stride
                o = out_p[l]
                s = lib.swa_rma_step(st_c[l], 1, r[0], r[1], r[2], r[3], sbase[l] + t * 16, q, q,
                                     nm_c[l], o[0], o[1], o[2], o[3], ws_p, ws_n, stream)
                assert s == 0
                if p in samples and l in CHECK_LAYERS:
                    captured[(p, l)] = [x.clone() for x in outs[l]]
            if (p + 1) % O.BLOCK == 0:
                c = p // O.BLOCK
                for l in range(L):
                    assert lib.rma_commit_topk(st_c[l], 1, keeps[c, l].data_ptr(), stream) == 0
        torch.cuda.synchronize()
        if c0 % (16 * CHUNK) == 0:
            print(f"stream at position {c0 + CHUNK}", flush=True)
    torch.cuda.synchronize()
    assert sum(t.numel() * t.element_size() for t in states[0].__dict__.values()) == state_bytes
    kg = keeps.cpu().numpy()
    print("stream done; checking", flush=True)

    # every layer: final bank = global best 1024 of all records of each group
    for l in range(L):
        allsc = np.concatenate([W.stream_scores_np(WL, l, c) for c in range(NBLK)])  # [T][4]
        src = np.arange(T)
        got_src = states[l].bank_src.cpu().numpy()[0]
        for g in range(4):
            order = np.lexsort((src, -allsc[:, g].astype(np.float64)))
            assert np.array_equal(np.sort(got_src[g]), np.sort(order[:O.BANK])), (l, g)
        assert int(states[l].n_bank[0]) == O.BANK and int(states[l].pos[0]) == T - 1

    snap_blocks = {p // O.BLOCK - 1 for p in SAMPLES if p >= O.BLOCK}
    for l in CHECK_LAYERS:
        k_ref, snaps = _oracle_chain(l, snap_blocks)
        assert np.array_equal(kg[:, l], k_ref), f"layer {l}: keep_idx differs"
        print(f"layer {l}: {NBLK} commits bit-exact", flush=True)
        g = gains[l]
        for p in SAMPLES:
            lo = max(0, p - O.WINDOW + 1)
            wpos = np.arange(lo, p + 1)
            slots = wpos % O.WINDOW
            wk = np.zeros((O.WINDOW, 4, 256), np.uint16)
            wv = np.zeros((O.WINDOW, 4, 256), np.uint16)
            wk[slots] = _oracle_keys(l, "k_win", g["gk_win"], wpos)
            wv[slots] = W.record_rows_np(WL, l, "v_win", wpos)
            n_w = min(p + 1, O.WINDOW)
            c = p // O.BLOCK
            ppos = np.arange(c * O.BLOCK, p + 1)
            pk = _oracle_keys(l, "k_rma", g["gk_rma"], ppos)
            pv = W.record_rows_np(WL, l, "v_rma", ppos)
            if c >= 1:
                bsrc, nb = snaps[c - 1]
            else:
                bsrc, nb = np.zeros((4, O.BANK), np.int32), 0
            keys, vals = [], []
            for gg in range(4):
                bk = _oracle_keys(l, "k_rma", g["gk_rma"], bsrc[gg, :nb])[:, gg] if nb else \
                    np.zeros((0, 256), np.uint16)
                bv = W.record_rows_np(WL, l, "v_rma", bsrc[gg, :nb])[:, gg] if nb else \
                    np.zeros((0, 256), np.uint16)
                keys.append(np.concatenate([bk, pk[:, gg]]))
                vals.append(np.concatenate([bv, pv[:, gg]]))
            q = W.stream_q_np(WL, l, p, p + 1)[0]
            ow, lw = O.decode_one([wk[:n_w, gg] for gg in range(4)], [wv[:n_w, gg] for gg in range(4)],
                                  q, g["gq_win"], p, WL.eps, WL.rope_base)
            orr, lr = O.decode_one(keys, vals, q, g["gq_rma"], p, WL.eps, WL.rope_base)
            o_w, l_w, o_r, l_r = captured[(p, l)]
            assert_attn_close(bits_host(o_w[0]), l_w[0].cpu().numpy(), ow, lw, what=f"p={p} l={l} win")
            assert_attn_close(bits_host(o_r[0]), l_r[0].cpu().numpy(), orr, lr, what=f"p={p} l={l} rma")

    # the scorer on sampled blocks of the stream's hidden states
    w1, w2 = W.scorer_weights(WL, 3)
    for c in (0, 511, NBLK - 1):
        h = W.stream_hidden_np(WL, 3, c * O.BLOCK, (c + 1) * O.BLOCK)
        out = torch.empty(O.BLOCK, 4, device=DEV)
        R.rma_score(bf16_dev(h), O.BLOCK, 2560, f32_dev(w1), f32_dev(w2), out, 4)
        torch.cuda.synchronize()
        assert_scores_close(out.cpu().numpy(), O.score(h, w1, w2), what=f"stream block {c}")
