"""The five synthetic workloads of the RMA hot path.

Each workload is named by what it is.  Sizes follow the EdgeRock-4B model as the
pages describe it: 16 query heads over 4 KV groups, head width 256, a 1024-slot
sliding window, a 1024-record anchor bank and a 256-record pending block per
group, 8 SWA||RMA layers, hidden width 2560 feeding a 2560->256->4 scorer.

* ``tiny_stream``       batch 1, one layer, 2048-token stream (8 commits), then
                        8 decode steps at positions 2048..2055.
* ``steady_b64``        batch 64, 8 layers, decode at position 32768 with full
                        window, full bank and a full pending block.
* ``headline_b512``     batch 512, 8 layers, decode at position 65536 (same
                        per-sequence state as ``steady_b64``; 36 GiB total),
                        norm gains N(1, 0.1).
* ``commit_burst_b512`` batch 512, 8 layers: score 256 new tokens per sequence
                        and merge them with a full bank, with about 5% exact
                        score ties planted.
* ``long_stream_b1``    batch 1, 8 layers, a stream to position 262143.
* ``gdn_decode_b512``   batch 512, the 24 Gated DeltaNet layers, one decode step at
                        position 65536 over FP16 recurrent matrices (12 GiB).
* ``gdn_decode_b1``     batch 1, the 24 GDN layers, FP32 matrices.
* ``headline_b512_fp8`` ``headline_b512`` with every stored K/V row held as 256
                        E4M3 codes and one FP32 scale: codes of N(0,1) quantiles
                        times 128 with scales in [3/512, 4/512), so a row decodes
                        to about N(0, 1) as in the BF16 state.
* ``headline_b512_i8``  ``headline_b512`` with every stored K/V row held as 256
                        signed 8-bit codes and one FP32 scale: N(0,1) quantiles
                        times 36, rounded and clipped to [-127, 127], with scales
                        in [3/128, 4/128), so a row again decodes to about N(0, 1).

Every large BF16 tensor is a counter-based stream (see ``synth.core``), so the
host can regenerate any slice of what the device drew.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .core import (
    StreamKey,
    distinct_ints_np,
    normal_bf16_at_np,
    normal_bf16_np,
    normal_bf16_torch_,
    normal_e4m3_np,
    normal_e4m3_torch_,
    normal_f32_np,
    normal_i8_np,
    normal_i8_torch_,
    rng_np,
    row_scale_np,
    row_scale_torch_,
    scaled_normal_np,
    scaled_normal_torch_,
    stream_key,
)

Q_HEADS = 16
KV_GROUPS = 4
HEAD_DIM = 256
WINDOW = 1024
BANK = 1024
BLOCK = 256
HIDDEN = 2560
MID = 256
LAYERS = 8

# Standard deviation of a 2560->256->4 bias-free chain with N(0,1) inputs and
# N(0, 0.02^2) weights: sqrt(256 * 2560 * 0.02^2 * 0.02^2) = 0.3238.
SCORE_STD = float(np.sqrt(256 * 2560 * 0.02**2 * 0.02**2))


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    layers: int
    position: int  # decode position (or stream length for the streams)
    gains: str  # "ones" or "normal"
    src_hi: int = 31744  # anchor source positions are drawn from [0, src_hi)
    eps: float = 1e-6
    rope_base: float = 1e7
    extra: dict = field(default_factory=dict)


TINY_STREAM = Workload("tiny_stream", batch=1, layers=1, position=2048, gains="normal",
                       extra={"decode_steps": 8})
STEADY_B64 = Workload("steady_b64", batch=64, layers=8, position=32768, gains="ones")
HEADLINE_B512 = Workload("headline_b512", batch=512, layers=8, position=65536, gains="normal")
COMMIT_BURST_B512 = Workload("commit_burst_b512", batch=512, layers=8, position=32767,
                             gains="ones", src_hi=32512)
LONG_STREAM_B1 = Workload("long_stream_b1", batch=1, layers=8, position=262144, gains="normal")
HEADLINE_B512_FP8 = Workload("headline_b512_fp8", batch=512, layers=8, position=65536,
                             gains="normal", extra={"kv": "e4m3"})
HEADLINE_B512_I8 = Workload("headline_b512_i8", batch=512, layers=8, position=65536,
                            gains="normal", extra={"kv": "int8"})

GDN_DECODE_B512 = Workload("gdn_decode_b512", batch=512, layers=24, position=65536, gains="ones",
                           extra={"state": "f16"})
GDN_DECODE_B1 = Workload("gdn_decode_b1", batch=1, layers=24, position=65536, gains="ones",
                         extra={"state": "f32"})
# GDN chunked prefill: one 256-token chunk per sequence at positions 65536.. (FP16 state)
GDN_PREFILL_B512 = Workload("gdn_prefill_b512", batch=512, layers=24, position=65536,
                            gains="ones", extra={"state": "f16", "chunk": 256})
# The same at batch 1 (FP32 state): the input phase of one long request
GDN_PREFILL_B1 = Workload("gdn_prefill_b1", batch=1, layers=24, position=65536,
                          gains="ones", extra={"state": "f32", "chunk": 256})

# Chunked prefill: one 256-token chunk per sequence at positions 65536..65791 on a
# steady-state layer (full window and bank, empty pending block).
PREFILL_B512 = Workload("prefill_b512", batch=512, layers=8, position=65535, gains="normal")
PREFILL_B64 = Workload("prefill_b64", batch=64, layers=8, position=65535, gains="normal")

WORKLOADS = {w.name: w for w in (TINY_STREAM, STEADY_B64, HEADLINE_B512, COMMIT_BURST_B512,
                                 LONG_STREAM_B1, HEADLINE_B512_FP8, HEADLINE_B512_I8, GDN_DECODE_B512,
                                 GDN_DECODE_B1, PREFILL_B512, PREFILL_B64, GDN_PREFILL_B512,
                                 GDN_PREFILL_B1)}


def key(wl: Workload | str, *names) -> StreamKey:
    return stream_key(wl if isinstance(wl, str) else wl.name, *names)


# ------------------------------------------------------------------ small tensors
def gains(wl: Workload, layer: int) -> dict:
    """The four FP32 [256] norm gains of one layer: gq_win, gk_win, gq_rma, gk_rma."""
    out = {}
    for nm in ("gq_win", "gk_win", "gq_rma", "gk_rma"):
        if wl.gains == "ones":
            out[nm] = np.ones(HEAD_DIM, np.float32)
        else:
            out[nm] = normal_f32_np(key(wl, layer, nm), (HEAD_DIM,), 1.0, 0.1)
    return out


def scorer_weights(wl: Workload, layer: int):
    """W1 FP32 [2560][256] and W2 FP32 [256][4], both N(0, 0.02^2)."""
    w1 = normal_f32_np(key(wl, layer, "W1"), (HIDDEN, MID), 0.0, 0.02)
    w2 = normal_f32_np(key(wl, layer, "W2"), (MID, KV_GROUPS), 0.0, 0.02)
    return w1, w2


# ------------------------------------------------------------------ decode state
KV_NAMES = ("win_k", "win_v", "bank_k", "bank_v", "pend_k", "pend_v")


def kv_slots(name: str) -> int:
    return {"win": WINDOW, "bank": BANK, "pend": BLOCK}[name.split("_")[0]]


def kv_np(wl: Workload, layer: int, name: str, b: int) -> np.ndarray:
    """One sequence's slice ``[4][slots][256]`` (uint16 BF16 bits) of a K/V state tensor."""
    per_seq = KV_GROUPS * kv_slots(name) * HEAD_DIM
    x = normal_bf16_np(key(wl, layer, name), per_seq, start=b * per_seq)
    return x.reshape(KV_GROUPS, kv_slots(name), HEAD_DIM)


def kv_torch_(wl: Workload, layer: int, name: str, out) -> None:
    """Fill the device tensor ``out`` ``[B][4][slots][256]`` with the same stream."""
    assert out.shape[1:] == (KV_GROUPS, kv_slots(name), HEAD_DIM)
    normal_bf16_torch_(out, key(wl, layer, name))


def kv_fp8_np(wl: Workload, layer: int, name: str, b: int):
    """One sequence's FP8 slice: codes ``[4][slots][256]`` (uint8) and scales ``[4][slots]``."""
    slots = kv_slots(name)
    per_seq = KV_GROUPS * slots
    codes = normal_e4m3_np(key(wl, layer, name, "e4m3"), per_seq * HEAD_DIM,
                           start=b * per_seq * HEAD_DIM)
    scales = row_scale_np(key(wl, layer, name, "scale"), per_seq, start=b * per_seq)
    return codes.reshape(KV_GROUPS, slots, HEAD_DIM), scales.reshape(KV_GROUPS, slots)


def kv_fp8_torch_(wl: Workload, layer: int, name: str, codes, scales) -> None:
    """Fill device tensors codes ``[B][4][slots][256]`` (uint8) and scales ``[B][4][slots]``."""
    assert codes.shape[1:] == (KV_GROUPS, kv_slots(name), HEAD_DIM)
    assert scales.shape == codes.shape[:3]
    normal_e4m3_torch_(codes, key(wl, layer, name, "e4m3"))
    row_scale_torch_(scales, key(wl, layer, name, "scale"))


def kv_i8_np(wl: Workload, layer: int, name: str, b: int):
    """One sequence's INT8 slice: codes ``[4][slots][256]`` (uint8 bytes of int8) and
    scales ``[4][slots]`` in [3/128, 4/128)."""
    slots = kv_slots(name)
    per_seq = KV_GROUPS * slots
    codes = normal_i8_np(key(wl, layer, name, "int8"), per_seq * HEAD_DIM,
                         start=b * per_seq * HEAD_DIM)
    scales = row_scale_np(key(wl, layer, name, "scale"), per_seq, start=b * per_seq, denom=128)
    return codes.reshape(KV_GROUPS, slots, HEAD_DIM), scales.reshape(KV_GROUPS, slots)


def kv_i8_torch_(wl: Workload, layer: int, name: str, codes, scales) -> None:
    """Fill device tensors codes ``[B][4][slots][256]`` (uint8) and scales ``[B][4][slots]``."""
    assert codes.shape[1:] == (KV_GROUPS, kv_slots(name), HEAD_DIM)
    assert scales.shape == codes.shape[:3]
    normal_i8_torch_(codes, key(wl, layer, name, "int8"))
    row_scale_torch_(scales, key(wl, layer, name, "scale"), denom=128)


def q_np(wl: Workload, layer: int, b: int, step: int = 0) -> np.ndarray:
    """Raw query ``[16][256]`` (uint16 BF16 bits) of sequence b."""
    per_seq = Q_HEADS * HEAD_DIM
    return normal_bf16_np(key(wl, layer, "q", step), per_seq, start=b * per_seq).reshape(
        Q_HEADS, HEAD_DIM)


def q_torch_(wl: Workload, layer: int, out, step: int = 0) -> None:
    normal_bf16_torch_(out, key(wl, layer, "q", step))


def bank_src(wl: Workload, layer: int, b: int) -> np.ndarray:
    """Source positions ``[4][1024]`` of a full bank: distinct per group, uniform in [0, src_hi)."""
    return np.stack([distinct_ints_np(key(wl, layer, "bank_src", b, g), BANK, 0, wl.src_hi)
                     for g in range(KV_GROUPS)])


def bank_src_all(wl: Workload, layer: int) -> np.ndarray:
    return np.stack([bank_src(wl, layer, b) for b in range(wl.batch)])


def pend_src(wl: Workload) -> np.ndarray:
    """Source positions ``[256]`` of a full pending block: the last 256 positions up to p."""
    return np.arange(wl.position - BLOCK + 1, wl.position + 1, dtype=np.int32)


def decode_meta(wl: Workload, layer: int) -> dict:
    """Host-side metadata of a steady-state layer (all sequences)."""
    B = wl.batch
    return {
        "bank_score": normal_f32_np(key(wl, layer, "bank_score"), (B, KV_GROUPS, BANK)),
        "bank_src": bank_src_all(wl, layer),
        "pend_score": normal_f32_np(key(wl, layer, "pend_score"), (B, BLOCK, KV_GROUPS)),
        "pend_src": np.broadcast_to(pend_src(wl), (B, BLOCK)).copy(),
        "n_bank": np.full(B, BANK, np.int32),
        "n_pend": np.full(B, BLOCK, np.int32),
        "pos": np.full(B, wl.position, np.int32),
    }


def decode_state_np(wl: Workload, layer: int, b: int) -> dict:
    """Everything the decode step of sequence b in one layer reads (host copy)."""
    st = {nm: kv_np(wl, layer, nm, b) for nm in KV_NAMES}
    st["n_bank"], st["n_pend"], st["pos"] = BANK, BLOCK, wl.position
    return st


# ------------------------------------------------------------------ commit burst
def burst_hidden_np(wl: Workload, layer: int, b: int, rows=None) -> np.ndarray:
    """Hidden states ``[256][2560]`` (BF16 bits) of sequence b's new block, with duplicated rows."""
    per_seq = BLOCK * HIDDEN
    h = normal_bf16_np(key(wl, layer, "H"), per_seq, start=b * per_seq).reshape(BLOCK, HIDDEN)
    for dst, src in burst_dup_rows(wl, layer)[b]:
        h[dst] = h[src]
    return h if rows is None else h[rows]


def burst_hidden_torch_(wl: Workload, layer: int, out) -> None:
    """Fill ``out`` ``[B][256][2560]`` on its device with the same hidden states."""
    import torch

    normal_bf16_torch_(out, key(wl, layer, "H"))
    dups = burst_dup_rows(wl, layer)
    bi = torch.tensor([b for b in range(wl.batch) for _ in dups[b]], dtype=torch.int64)
    di = torch.tensor([d for b in range(wl.batch) for d, _ in dups[b]], dtype=torch.int64)
    si = torch.tensor([s for b in range(wl.batch) for _, s in dups[b]], dtype=torch.int64)
    bi, di, si = bi.to(out.device), di.to(out.device), si.to(out.device)
    out[bi, di] = out[bi, si]


def burst_dup_rows(wl: Workload, layer: int, frac: float = 0.025):
    """Per sequence, (dst, src) row pairs: 2.5% of the block's rows copy another row."""
    rng = rng_np(key(wl, layer, "dup_rows"))
    n = int(frac * BLOCK)
    out = []
    for _ in range(wl.batch):
        pick = rng.choice(BLOCK, size=2 * n, replace=False)
        out.append([(int(d), int(s)) for d, s in zip(pick[:n], pick[n:])])
    return out


def burst_scores(wl: Workload, layer: int) -> dict:
    """Commit inputs with planted exact ties (host; FP32).

    Per (sequence, group) the 1280 candidate scores are drawn N(0, 0.3238^2),
    sorted, and the eight values around the 1024th place are set equal so the
    cut falls inside a run of ties; in every fourth segment the whole segment
    is shifted so that run is exactly zero, with half of it written as -0.0.
    The values are then shuffled into 1024 bank and 256 pending slots.  After
    that, 2.5% of each sequence's pending rows copy another row (all groups),
    and 2.5% of each segment's bank scores copy a pending score.
    Returns bank_score [B][4][1024], pend_score [B][256][4] and the sources.
    """
    B, G = wl.batch, KV_GROUPS
    rng = rng_np(key(wl, layer, "burst_scores"))
    n = BANK + BLOCK
    v = np.sort(rng.standard_normal((B, G, n)) * SCORE_STD, axis=-1)[..., ::-1].copy()
    v[..., BANK - 4:BANK + 4] = v[..., BANK - 1:BANK]
    zseg = (np.arange(B * G).reshape(B, G) % 4) == 3
    v[zseg] -= v[zseg][:, BANK - 1:BANK]
    v = v.astype(np.float32)
    neg = v[zseg]
    neg[:, BANK - 4:BANK] = -0.0
    neg[:, BANK:BANK + 4] = 0.0
    v[zseg] = neg
    perm = np.argsort(rng.random((B, G, n)), axis=-1)
    v = np.take_along_axis(v, perm, axis=-1)
    bank_score = v[..., :BANK].copy()
    pend_score = np.ascontiguousarray(v[..., BANK:].transpose(0, 2, 1))  # [B][256][4]
    nd = int(0.025 * BLOCK)
    for b in range(B):
        pick = rng.choice(BLOCK, size=2 * nd, replace=False)
        pend_score[b, pick[:nd]] = pend_score[b, pick[nd:]]
    nb = int(round(0.025 * BANK))
    for b in range(B):
        for g in range(G):
            dst = rng.choice(BANK, size=nb, replace=False)
            src = rng.integers(0, BLOCK, size=nb)
            bank_score[b, g, dst] = pend_score[b, src, g]
    return {
        "bank_score": bank_score,
        "pend_score": pend_score,
        "bank_src": bank_src_all(wl, layer),
        "pend_src": np.broadcast_to(pend_src(wl), (B, BLOCK)).copy(),
        "n_bank": np.full(B, BANK, np.int32),
        "n_pend": np.full(B, BLOCK, np.int32),
        "pos": np.full(B, wl.position, np.int32),
    }



def plant_burst_ties(wl: Workload, layer: int, pend_score) -> dict:
    """Commit inputs built around given pending scores (e.g. the scorer's output on
    the burst's hidden rows, whose duplicated rows already give equal score rows).

    pend_score is FP32 [B][256][4].  Per (sequence, group): bank scores are drawn
    N(0, s^2) with s the standard deviation of the given scores; 2.5% of them copy
    a pending score of the same group; then the 1280 values are ranked and the
    eight around the 1024th place are set equal to the 1024th, so the cut falls
    inside a run of ties; in every fourth segment the 1024th value is subtracted
    from all 1280 (an order-preserving FP32 shift) and the run is written as four
    -0.0 and four +0.0.  Only values change, never ranks outside the run.
    Returns the same fields as burst_scores.
    """
    B, G = wl.batch, KV_GROUPS
    ps = np.array(pend_score, np.float32, copy=True).reshape(B, BLOCK, G)
    rng = rng_np(key(wl, layer, "planted_ties"))
    std = float(ps.astype(np.float64).std())
    bank_score = (rng.standard_normal((B, G, BANK)) * std).astype(np.float32)
    nb = int(round(0.025 * BANK))
    for b in range(B):
        for g in range(G):
            dst = rng.choice(BANK, size=nb, replace=False)
            src = rng.integers(0, BLOCK, size=nb)
            bank_score[b, g, dst] = ps[b, src, g]
    for b in range(B):
        for g in range(G):
            v = np.concatenate([bank_score[b, g], ps[b, :, g]])
            order = np.argsort(-v.astype(np.float64), kind="stable")
            run = order[BANK - 4:BANK + 4]
            v[run] = v[order[BANK - 1]]
            if (b * G + g) % 4 == 3:
                v = (v - v[order[BANK - 1]]).astype(np.float32)
                v[run[:4]] = -0.0
                v[run[4:]] = 0.0
            bank_score[b, g] = v[:BANK]
            ps[b, :, g] = v[BANK:]
    return {
        "bank_score": bank_score,
        "pend_score": ps,
        "bank_src": bank_src_all(wl, layer),
        "pend_src": np.broadcast_to(pend_src(wl), (B, BLOCK)).copy(),
        "n_bank": np.full(B, BANK, np.int32),
        "n_pend": np.full(B, BLOCK, np.int32),
        "pos": np.full(B, wl.position, np.int32),
    }

# ------------------------------------------------------------------ token streams
RECORD_NAMES = ("k_win", "v_win", "k_rma", "v_rma")


def record_np(wl: Workload, layer: int, name: str, t0: int, t1: int) -> np.ndarray:
    """Raw per-token records ``[t1-t0][4][256]`` (BF16 bits) of positions t0..t1-1 (batch 1)."""
    per_tok = KV_GROUPS * HEAD_DIM
    x = normal_bf16_np(key(wl, layer, "rec", name), (t1 - t0) * per_tok, start=t0 * per_tok)
    return x.reshape(t1 - t0, KV_GROUPS, HEAD_DIM)


def record_rows_np(wl: Workload, layer: int, name: str, positions) -> np.ndarray:
    """Raw records ``[len(positions)][4][256]`` at arbitrary positions (batch 1)."""
    per_tok = KV_GROUPS * HEAD_DIM
    pos = np.asarray(positions, dtype=np.uint64)
    idx = pos[:, None] * np.uint64(per_tok) + np.arange(per_tok, dtype=np.uint64)[None, :]
    return normal_bf16_at_np(key(wl, layer, "rec", name), idx).reshape(len(pos), KV_GROUPS,
                                                                       HEAD_DIM)


def record_torch_(wl: Workload, layer: int, name: str, t0: int, out) -> None:
    normal_bf16_torch_(out, key(wl, layer, "rec", name), start=t0 * KV_GROUPS * HEAD_DIM)


def stream_q_np(wl: Workload, layer: int, t0: int, t1: int) -> np.ndarray:
    """Raw queries ``[t1-t0][16][256]`` of positions t0..t1-1 (batch 1)."""
    per_tok = Q_HEADS * HEAD_DIM
    x = normal_bf16_np(key(wl, layer, "stream_q"), (t1 - t0) * per_tok, start=t0 * per_tok)
    return x.reshape(t1 - t0, Q_HEADS, HEAD_DIM)


def stream_q_torch_(wl: Workload, layer: int, t0: int, out) -> None:
    normal_bf16_torch_(out, key(wl, layer, "stream_q"), start=t0 * Q_HEADS * HEAD_DIM)


def stream_hidden_np(wl: Workload, layer: int, t0: int, t1: int) -> np.ndarray:
    """Hidden states ``[t1-t0][2560]`` of positions t0..t1-1 (batch 1)."""
    x = normal_bf16_np(key(wl, layer, "stream_H"), (t1 - t0) * HIDDEN, start=t0 * HIDDEN)
    return x.reshape(t1 - t0, HIDDEN)


def stream_hidden_torch_(wl: Workload, layer: int, t0: int, out) -> None:
    normal_bf16_torch_(out, key(wl, layer, "stream_H"), start=t0 * HIDDEN)


def stream_scores_np(wl: Workload, layer: int, block: int) -> np.ndarray:
    """Generator-supplied candidate scores ``[256][4]`` (FP32) of one 256-token block."""
    return normal_f32_np(key(wl, layer, "stream_score", block), (BLOCK, KV_GROUPS), 0.0,
                         SCORE_STD)


def prefill_record_np(wl: Workload, layer: int, name: str, b: int, chunk: int) -> np.ndarray:
    """Raw chunk records ``[chunk][4][256]`` (BF16 bits) of sequence b."""
    per = chunk * KV_GROUPS * HEAD_DIM
    return normal_bf16_np(key(wl, layer, "prefill", name), per, start=b * per).reshape(
        chunk, KV_GROUPS, HEAD_DIM)


def prefill_record_torch_(wl: Workload, layer: int, name: str, out) -> None:
    """All sequences' chunk records ``[B][chunk][4][256]``."""
    normal_bf16_torch_(out, key(wl, layer, "prefill", name))


def prefill_q_np(wl: Workload, layer: int, b: int, chunk: int) -> np.ndarray:
    """Raw chunk queries ``[chunk][16][256]`` (BF16 bits) of sequence b."""
    per = chunk * Q_HEADS * HEAD_DIM
    return normal_bf16_np(key(wl, layer, "prefill", "q"), per, start=b * per).reshape(
        chunk, Q_HEADS, HEAD_DIM)


def prefill_q_torch_(wl: Workload, layer: int, out) -> None:
    normal_bf16_torch_(out, key(wl, layer, "prefill", "q"))


# ------------------------------------------------------------------ GDN decode step
# The pages give no activations or weights for the recurrent layers; the draws are
# unit-scale: projected inputs N(0,1) (BF16), gate inputs N(0,1), convolution taps
# N(0, 0.5^2), A = exp(A_log) uniform in [1, 16), dt_bias N(0,1), and recurrent
# matrices N(0, 1/64) -- the spread a unit-key delta rule reaches with values of
# spread about 0.5 under moderate decay.
GDN_V_HEADS, GDN_K_HEADS, GDN_DIM, GDN_CONV, GDN_CONV_DIM = 32, 16, 128, 4, 8192
GDN_S_SCALE = 0.125  # a power of two: the FP16 and FP32 draws are exact scalings


def gdn_state_np(wl: Workload, layer: int, b: int, h: int) -> np.ndarray:
    """Recurrent matrix ``[128][128]`` of sequence b, value head h (float16 or float32)."""
    per = GDN_DIM * GDN_DIM
    dt = np.float16 if wl.extra["state"] == "f16" else np.float32
    return scaled_normal_np(key(wl, layer, "S"), per, start=(b * GDN_V_HEADS + h) * per,
                            scale=GDN_S_SCALE, dtype=dt).reshape(GDN_DIM, GDN_DIM)


def gdn_state_torch_(wl: Workload, layer: int, out) -> None:
    scaled_normal_torch_(out, key(wl, layer, "S"), scale=GDN_S_SCALE)


def gdn_conv_np(wl: Workload, layer: int, b: int) -> np.ndarray:
    """Convolution ring ``[4][8192]`` (BF16 bits) of sequence b."""
    per = GDN_CONV * GDN_CONV_DIM
    return normal_bf16_np(key(wl, layer, "conv"), per, start=b * per).reshape(GDN_CONV,
                                                                              GDN_CONV_DIM)


def gdn_conv_torch_(wl: Workload, layer: int, out) -> None:
    normal_bf16_torch_(out, key(wl, layer, "conv"))


def gdn_x_np(wl: Workload, layer: int, b: int, step: int = 0) -> np.ndarray:
    """Projected input ``[8192]`` (BF16 bits) of sequence b."""
    return normal_bf16_np(key(wl, layer, "x", step), GDN_CONV_DIM, start=b * GDN_CONV_DIM)


def gdn_x_torch_(wl: Workload, layer: int, out, step: int = 0) -> None:
    normal_bf16_torch_(out, key(wl, layer, "x", step))


def gdn_chunk_x_torch_(wl: Workload, layer: int, out) -> None:
    """A chunk's projected inputs ``[B][C][8192]`` (BF16)."""
    normal_bf16_torch_(out, key(wl, layer, "chunk_x"))


def gdn_chunk_x_np(wl: Workload, layer: int, b: int, chunk: int) -> np.ndarray:
    per = chunk * GDN_CONV_DIM
    return normal_bf16_np(key(wl, layer, "chunk_x"), per, start=b * per).reshape(chunk,
                                                                                 GDN_CONV_DIM)


def gdn_chunk_gates(wl: Workload, layer: int, chunk: int):
    """a, b ``[B][C][32]`` FP32 (host) of a chunk."""
    return (normal_f32_np(key(wl, layer, "chunk_a"), (wl.batch, chunk, GDN_V_HEADS)),
            normal_f32_np(key(wl, layer, "chunk_b"), (wl.batch, chunk, GDN_V_HEADS)))


def gdn_gate_inputs(wl: Workload, layer: int, step: int = 0):
    """a, b ``[B][32]`` FP32 (host)."""
    return (normal_f32_np(key(wl, layer, "a", step), (wl.batch, GDN_V_HEADS)),
            normal_f32_np(key(wl, layer, "b", step), (wl.batch, GDN_V_HEADS)))


def gdn_params(wl: Workload, layer: int) -> dict:
    """conv_w ``[8192][4]``, a_log ``[32]``, dt_bias ``[32]`` (FP32, host)."""
    u = rng_np(key(wl, layer, "A")).uniform(1.0, 16.0, GDN_V_HEADS)
    return {
        "conv_w": normal_f32_np(key(wl, layer, "conv_w"), (GDN_CONV_DIM, GDN_CONV), 0.0, 0.5),
        "a_log": np.log(u).astype(np.float32),
        "dt_bias": normal_f32_np(key(wl, layer, "dt_bias"), (GDN_V_HEADS,)),
    }
