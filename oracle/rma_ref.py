"""Float64 reference of the Rock Memory Anchors (RMA) hot path of EdgeRock-4B.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code,
header, table or helper with the HIP path.

Every step here is an exact computation with a plain definition (RMS
normalisation, rotary embedding, softmax attention, a two-matrix product,
a top-k under a total order), so each function is that definition written out
in float64 with NumPy, looping over sequences, branches and heads.

Sources (web pages about EdgeRock-4B; cited by page and section):
  [FB]   fluxbbs.com, "EdgeRock-4B 开源：72 MiB 固定 KV，AIME 82.9 分"
         [FB §Mem]  section "72 MiB 是怎么算出来的" (state inventory, sizes, precisions)
         [FB §Arch] section "架构：递归、局部窗口与记忆锚点三件套" (layer pattern,
                    RMA write and read, norms, partial rotary, config values)
         [FB §FAQ]  section "常见问题"
  [QB]   neodrop.ai repost of the QbitAI article "内存还会跌吗？KV Cache砍掉99%，
         单卡吞吐飙6倍，港科大、CMU联手岩山科技开源新模型"
         [QB §Mech] section "三段记忆，只记值得记的" (one candidate per token,
                    merge every 256, top 1024 per KV group, immutable anchors)
         [QB §Thr]  section "为什么越贵" / "一张卡，512 路长推理"
  [GH]   agentlenshq.com, "rockmatrix-ai/EdgeRock", section "架构概览"
         (layer pattern, window 31.97 MiB, bank 32 MiB + pending 8 MiB)

Readings where the pages leave a step open (each is the plainest reading the
rest supports; the values are runtime parameters where possible):
  * RMSNorm: y = x / sqrt(mean(x^2) + eps) * gamma over one head's 256 dims,
    eps = 1e-6, one gain vector per branch shared by all heads (q) or groups (k).
  * Rotary: NeoX "rotate-half" pairing (i, i+32) inside dims 0..63,
    theta_i = base^(-2i/64), angle = position * theta_i, applied after the norm.
  * Keys are normalised and rotated once, when written, at their own position;
    values are stored raw.  The query is normalised and rotated at the current
    position on every read.
  * Head h reads KV group floor(h/4); softmax scale 1/sqrt(256) = 1/16; no
    soft-cap, sink or bias.
  * The anchor branch reads the committed bank followed by the pending block,
    under one softmax; the window branch reads the valid ring slots.  The two
    branches are returned separately with their log-sum-exps (the pages say the
    branches run in parallel but not how they are combined).
  * A token is appended before it attends.
  * The scorer chain has no nonlinearity between its two stages.
  * Selection order: higher score first; equal scores keep the lower source
    position; -0.0 equals +0.0; NaN ranks below every number.
  * Bank slots are slot-stable: survivors keep their slot, admitted pending
    records fill the free slots (evicted slots and never-used slots) in
    ascending slot order, taken in ascending pending order.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# Geometry [FB §Mem], [FB §Arch], [QB §Mech].
Q_HEADS = 16
KV_GROUPS = 4
HEAD_DIM = 256
ROPE_DIMS = 64
WINDOW = 1024
BANK = 1024
BLOCK = 256
HIDDEN = 2560
SCORER_MID = 256
RMA_LAYERS = 8
BF16_BYTES = 2

__all__ = [
    "Q_HEADS", "KV_GROUPS", "HEAD_DIM", "ROPE_DIMS", "WINDOW", "BANK", "BLOCK", "HIDDEN",
    "SCORER_MID", "RMA_LAYERS",
    "bf16_to_f64", "f64_to_bf16", "rms_norm", "rope", "rope_angles", "attend", "merge_lse",
    "LayerState", "new_layer_state", "append", "decode", "decode_one", "score", "commit",
    "commit_segment", "ordering_key", "kv_bytes_per_sequence", "window_bytes_per_sequence",
    "bank_bytes_per_sequence", "pending_bytes_per_sequence", "metadata_bytes_per_sequence",
    "source_kv_bytes_per_token",
]


# ---------------------------------------------------------------- BF16 codec
def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of BF16 bit patterns: the pattern is the top half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 to BF16 (8 significant bits, binary32 exponent range), nearest-even.

    Rounding is done once, directly from float64: the quantum is
    2^(e-8) for |x| in [2^(e-1), 2^e) and 2^-133 below the normal range.
    NaN becomes the canonical quiet NaN 0x7FC0; magnitudes that round to 2^128
    or beyond become infinities.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    nan = np.isnan(x)
    fin = np.isfinite(x)
    _, e = np.frexp(np.where(fin, x, 1.0))
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(np.where(fin, x, 0.0) / q) * q  # np.rint rounds half to even
    r = np.where(np.abs(r) >= 2.0**128, np.copysign(np.inf, r), r)
    r = np.where(fin, r, x)
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[...] = bits
    out[nan] = 0x7FC0
    return out


# ---------------------------------------------------------------- norm + rotary
def rms_norm(x, gamma, eps: float) -> np.ndarray:
    """Learned RMS normalisation of q and k over one head's 256 dims [FB §Arch].

    y_i = x_i / sqrt(mean_j x_j^2 + eps) * gamma_i.
    """
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, np.float64)


def rope_angles(pos: int, base: float, rot: int = ROPE_DIMS) -> np.ndarray:
    """Angles pos * base^(-2i/rot), i = 0..rot/2-1 (base 1e7 over 64 dims [FB §Arch])."""
    i = np.arange(rot // 2, dtype=np.float64)
    return float(pos) * np.power(float(base), -2.0 * i / rot)


def rope(x, pos: int, base: float, rot: int = ROPE_DIMS) -> np.ndarray:
    """Partial rotary embedding on dims 0..rot-1, pairs (i, i + rot/2); other dims untouched.

    [FB §Arch]: rotary acts on 64 of the 256 dims with base 10^7; values are not rotated.
    """
    x = np.asarray(x, np.float64)
    half = rot // 2
    phi = rope_angles(pos, base, rot)
    c, s = np.cos(phi), np.sin(phi)
    y = x.copy()
    a, b = x[..., :half], x[..., half:rot]
    y[..., :half] = a * c - b * s
    y[..., half:rot] = b * c + a * s
    return y


# ---------------------------------------------------------------- attention
def attend(qhat, keys, vals):
    """Softmax attention of query rows over key/value rows, scale 1/sqrt(d).

    Returns (o [m][d] float64, lse [m] float64) with lse the natural-log
    log-sum-exp of the scaled scores.  With no keys: o = 0 and lse = -inf.
    """
    qhat = np.asarray(qhat, np.float64)
    keys = np.asarray(keys, np.float64)
    vals = np.asarray(vals, np.float64)
    m_rows, d = qhat.shape
    if keys.shape[0] == 0:
        return np.zeros((m_rows, vals.shape[-1])), np.full(m_rows, -np.inf)
    s = (qhat @ keys.T) / math.sqrt(d)
    mx = s.max(axis=1, keepdims=True)
    w = np.exp(s - mx)
    den = w.sum(axis=1, keepdims=True)
    o = (w @ vals) / den
    lse = (mx + np.log(den))[:, 0]
    return o, lse


def merge_lse(o1, lse1, o2, lse2):
    """Combine two softmax results over disjoint key sets into the result over their union."""
    lse = np.logaddexp(lse1, lse2)
    w1 = np.where(np.isneginf(lse1), 0.0, np.exp(lse1 - lse))
    w2 = np.where(np.isneginf(lse2), 0.0, np.exp(lse2 - lse))
    return o1 * w1[:, None] + o2 * w2[:, None], lse


# ---------------------------------------------------------------- per-layer state
@dataclass
class LayerState:
    """One SWA||RMA layer's persistent attention state for B sequences [FB §Mem].

    K/V arrays hold BF16 bit patterns (uint16).  Slots [0, n_bank) of the bank
    and [0, n_pend) of the pending block are valid; window slot = position mod W.
    """

    win_k: np.ndarray  # [B][G][W][D]
    win_v: np.ndarray
    bank_k: np.ndarray  # [B][G][K][D]
    bank_v: np.ndarray
    bank_score: np.ndarray  # f32 [B][G][K]
    bank_src: np.ndarray  # i32 [B][G][K]
    pend_k: np.ndarray  # [B][G][P][D]
    pend_v: np.ndarray
    pend_score: np.ndarray  # f32 [B][P][G]
    pend_src: np.ndarray  # i32 [B][P]
    n_bank: np.ndarray  # i32 [B]
    n_pend: np.ndarray  # i32 [B]
    pos: np.ndarray  # i32 [B], newest appended position, -1 = none

    @property
    def window(self):
        return self.win_k.shape[2]

    @property
    def bank(self):
        return self.bank_k.shape[2]

    @property
    def block(self):
        return self.pend_k.shape[2]

    def copy(self) -> "LayerState":
        return LayerState(**{k: np.array(v, copy=True) for k, v in self.__dict__.items()})


def new_layer_state(batch: int, window: int = WINDOW, bank: int = BANK, block: int = BLOCK,
                    groups: int = KV_GROUPS, head_dim: int = HEAD_DIM) -> LayerState:
    z = lambda *s: np.zeros(s, np.uint16)  # noqa: E731
    return LayerState(
        win_k=z(batch, groups, window, head_dim), win_v=z(batch, groups, window, head_dim),
        bank_k=z(batch, groups, bank, head_dim), bank_v=z(batch, groups, bank, head_dim),
        bank_score=np.zeros((batch, groups, bank), np.float32),
        bank_src=np.zeros((batch, groups, bank), np.int32),
        pend_k=z(batch, groups, block, head_dim), pend_v=z(batch, groups, block, head_dim),
        pend_score=np.zeros((batch, block, groups), np.float32),
        pend_src=np.zeros((batch, block), np.int32),
        n_bank=np.zeros(batch, np.int32), n_pend=np.zeros(batch, np.int32),
        pos=np.full(batch, -1, np.int32),
    )


# ---------------------------------------------------------------- append (write side)
def append(st: LayerState, k_win, v_win, k_rma, v_rma, gk_win, gk_rma, eps: float,
           base: float, score=None) -> None:
    """Append the next token of every sequence to the window and the pending block.

    The writer emits one candidate record per token [QB §Mech].  Keys are RMS
    normalised with their branch's gain and rotated at the token's position;
    values are copied raw [FB §Arch].  Records are BF16 [FB §Mem].
    Inputs are BF16 bits [B][G][D]; ``score`` (optional) is FP32 [B][G].
    """
    B = st.pos.shape[0]
    for b in range(B):
        p = int(st.pos[b]) + 1
        t = int(st.n_pend[b])
        assert t < st.block, "pending block is full: commit before appending"
        slot = p % st.window
        for g in range(st.win_k.shape[1]):
            kw = rope(rms_norm(bf16_to_f64(k_win[b, g]), gk_win, eps), p, base)
            kr = rope(rms_norm(bf16_to_f64(k_rma[b, g]), gk_rma, eps), p, base)
            st.win_k[b, g, slot] = f64_to_bf16(kw)
            st.win_v[b, g, slot] = v_win[b, g]
            st.pend_k[b, g, t] = f64_to_bf16(kr)
            st.pend_v[b, g, t] = v_rma[b, g]
        st.pend_src[b, t] = p
        if score is not None:
            st.pend_score[b, t, :] = np.asarray(score, np.float32)[b]
        st.n_pend[b] = t + 1
        st.pos[b] = p


# ---------------------------------------------------------------- decode (read side)
def _branch_keys(st: LayerState, b: int, g: int, branch: str):
    if branch == "win":
        n = min(int(st.pos[b]) + 1, st.window)
        return st.win_k[b, g, :n], st.win_v[b, g, :n]
    nb, npd = int(st.n_bank[b]), int(st.n_pend[b])
    k = np.concatenate([st.bank_k[b, g, :nb], st.pend_k[b, g, :npd]])
    v = np.concatenate([st.bank_v[b, g, :nb], st.pend_v[b, g, :npd]])
    return k, v


def decode_one(keys_by_group, vals_by_group, q_bits, gamma_q, pos: int, eps: float,
               base: float):
    """One branch of one sequence: 16 query heads over 4 KV groups [FB §Arch].

    ``keys_by_group[g]``/``vals_by_group[g]`` are BF16 bit arrays [n_g][256].
    Returns o [16][256] float64 and lse [16] float64.
    """
    H = q_bits.shape[0]
    G = len(keys_by_group)
    per = H // G
    o = np.zeros((H, q_bits.shape[1]))
    lse = np.zeros(H)
    for g in range(G):
        K = bf16_to_f64(keys_by_group[g])
        V = bf16_to_f64(vals_by_group[g])
        for h in range(g * per, (g + 1) * per):
            qh = rope(rms_norm(bf16_to_f64(q_bits[h]), gamma_q, eps), pos, base)
            oh, lh = attend(qh[None, :], K, V)
            o[h], lse[h] = oh[0], lh[0]
    return o, lse


def decode(st: LayerState, q_win, q_rma, gq_win, gq_rma, eps: float, base: float):
    """The decode-step attention of one SWA||RMA layer for every sequence.

    Window branch: the current token's queries over the valid sliding-window
    slots.  Anchor branch: the same heads over the committed bank followed by
    the pending block [FB §Arch], [FB §Mem].  Returns
    (o_win [B][16][256], lse_win [B][16], o_rma, lse_rma), all float64.
    """
    B = st.pos.shape[0]
    G = st.win_k.shape[1]
    out = {}
    for branch, q, gq in (("win", q_win, gq_win), ("rma", q_rma, gq_rma)):
        o = np.zeros((B, Q_HEADS, HEAD_DIM))
        lse = np.zeros((B, Q_HEADS))
        for b in range(B):
            kv = [_branch_keys(st, b, g, branch) for g in range(G)]
            o[b], lse[b] = decode_one([k for k, _ in kv], [v for _, v in kv], q[b],
                                      gq, int(st.pos[b]), eps, base)
        out[branch] = (o, lse)
    return out["win"][0], out["win"][1], out["rma"][0], out["rma"][1]


# ---------------------------------------------------------------- scorer
def score(hidden_bits, w1, w2) -> np.ndarray:
    """Retention priorities: the bias-free FP32 chain 2560 -> 256 -> 4 [FB §Arch].

    s = (H W1) W2 in float64 from the exact BF16 inputs and FP32 weights, one
    column per KV group, rounded once to FP32.
    """
    h = bf16_to_f64(hidden_bits)
    z = h @ np.asarray(w1, np.float64)
    return (z @ np.asarray(w2, np.float64)).astype(np.float32)


# ---------------------------------------------------------------- commit
def ordering_key(score_value: float, src: int):
    """Sort key for "better first": higher score, then lower source position.

    -0.0 and +0.0 compare equal as Python floats; NaN sorts after every number.
    """
    s = float(score_value)
    if math.isnan(s):
        return (1, 0.0, int(src))
    return (0, -s, int(src))


def commit_segment(bank_score, bank_src, n_bank: int, pend_score, pend_src, n_pend: int,
                   cap: int):
    """Keep the best ``cap`` of a group's committed + pending records [QB §Mech], [FB §Arch].

    Returns (keep_idx [cap] int32, moves) where keep_idx[s] is s for a bank
    record that stays in slot s, cap + t for pending record t written into
    slot s, and -1 for an empty slot; ``moves`` lists (t, s) copies.
    """
    cands = [(ordering_key(bank_score[s], bank_src[s]), s) for s in range(n_bank)]
    cands += [(ordering_key(pend_score[t], pend_src[t]), cap + t) for t in range(n_pend)]
    cands.sort()
    kept = {idx for _, idx in cands[:min(cap, len(cands))]}
    keep_idx = np.full(cap, -1, np.int32)
    free = []
    for s in range(cap):
        if s < n_bank and s in kept:
            keep_idx[s] = s
        else:
            free.append(s)
    admitted = [t for t in range(n_pend) if cap + t in kept]
    moves = list(zip(admitted, free))
    for t, s in moves:
        keep_idx[s] = cap + t
    return keep_idx, moves


def commit(st: LayerState) -> np.ndarray:
    """Commit the pending block of every sequence; each KV group selects on its own.

    Groups are independent and may keep the same source positions [FB §Arch];
    kept records are copied once and never modified [QB §Mech].  Afterwards
    n_bank = min(cap, n_bank + n_pend) and n_pend = 0.  Returns keep_idx
    [B][G][cap] int32.
    """
    B, G, cap = st.bank_k.shape[0], st.bank_k.shape[1], st.bank
    keep = np.full((B, G, cap), -1, np.int32)
    for b in range(B):
        nb, npd = int(st.n_bank[b]), int(st.n_pend[b])
        for g in range(G):
            ki, moves = commit_segment(st.bank_score[b, g], st.bank_src[b, g], nb,
                                       st.pend_score[b, :, g], st.pend_src[b], npd, cap)
            keep[b, g] = ki
            for t, s in moves:
                st.bank_k[b, g, s] = st.pend_k[b, g, t]
                st.bank_v[b, g, s] = st.pend_v[b, g, t]
                st.bank_score[b, g, s] = st.pend_score[b, t, g]
                st.bank_src[b, g, s] = st.pend_src[b, t]
        st.n_bank[b] = min(cap, nb + npd)
        st.n_pend[b] = 0
    return keep


# ---------------------------------------------------------------- closed forms [FB §Mem]
def bank_bytes_per_sequence(layers=RMA_LAYERS, groups=KV_GROUPS, bank=BANK, d=HEAD_DIM):
    """Committed anchors: key and value x layers x groups x records x head width x 2 B."""
    return 2 * layers * groups * bank * d * BF16_BYTES


def pending_bytes_per_sequence(layers=RMA_LAYERS, groups=KV_GROUPS, block=BLOCK, d=HEAD_DIM):
    return 2 * layers * groups * block * d * BF16_BYTES


def window_bytes_per_sequence(layers=RMA_LAYERS, groups=KV_GROUPS, window=WINDOW, d=HEAD_DIM):
    return 2 * layers * groups * window * d * BF16_BYTES


def kv_bytes_per_sequence(**kw):
    """Attention K/V state per sequence: window + bank + pending, independent of length."""
    return window_bytes_per_sequence() + bank_bytes_per_sequence() + pending_bytes_per_sequence()


def metadata_bytes_per_sequence(layers=RMA_LAYERS, groups=KV_GROUPS, bank=BANK, block=BLOCK):
    """Per-record bookkeeping: FP32 score + int32 source per bank record and group, and
    per pending token one FP32 score per group plus one int32 source."""
    return layers * (groups * bank * (4 + 4) + block * (groups * 4 + 4))


def source_kv_bytes_per_token(layers=RMA_LAYERS, kv_heads=KV_GROUPS, d=HEAD_DIM):
    """Full-attention KV growth of a model with the same 8 attention layers, 4 KV heads,
    head width 256 and BF16 cache: key + value per layer per head per token."""
    return 2 * layers * kv_heads * d * BF16_BYTES
