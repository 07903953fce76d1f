"""Float64 reference of the FP8 K/V state variant of the RMA hot path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with the
HIP path.

The pages list quantised releases of EdgeRock-4B's weights (fluxbbs.com page, section
"架构：递归、局部窗口与记忆锚点三件套"; neodrop.ai repost of the QbitAI article, section
"开源到哪一步") but no format for the attention state itself, so this variant is a
reading of this build:

  * every stored K and V row (the 256 values of one sequence, KV group and slot) is
    held as 256 OCP FP8 E4M3 codes and one FP32 scale;
  * scale = amax / 448 with amax = max_i |x_i| (448 is the largest finite E4M3
    value), computed in FP32; a row whose amax is below 448 * 2^-126 (where
    448 / amax would pass 2^126 and the scale would leave the normal FP32 range),
    the all-zero row included, has scale 0 and all codes 0;
  * code_i = E4M3(fp32(x_i * inv)), inv = fp32(448 / amax), rounding to nearest,
    ties to even;
  * the stored row means code_value_i * scale.

Keys are quantised from their FP32 normalised and rotated value (the value the BF16
path rounds to BF16); values from their BF16 input.  The quantisation decides
integer codes, so it runs in FP32 with the operations the kernels use (both
sides take that decision in the same precision); everything after dequantisation
is float64 as in the BF16 oracle.  Attention, commit selection and bank layout are
those of ``oracle.rma_ref`` applied to the dequantised rows: the selection never
reads K/V, and an admitted row moves with its codes and scale unchanged.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import rma_ref as R

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


# ---------------------------------------------------------------- E4M3 codec
def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3 (no infinities): sign bit, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 holds subnormals m * 2^-9; S.1111.111 is NaN."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code, ties to even.  |x| > 464 (past the midpoint between 448
    and the next step, 480, which the format lacks) and NaN give NaN codes; 464
    itself is a tie and goes to the even neighbour, 448."""
    x = np.asarray(x, np.float64)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    a = np.abs(x)
    out = np.zeros(x.shape, np.int64)
    nan = np.isnan(a) | (a > 464.0)
    # subnormal range: a < 2^-6 -> multiples of 2^-9 (8 * 2^-9 is the smallest normal)
    sub = ~nan & (a < 2.0 ** -6)
    ms = np.rint(np.minimum(a, 1.0) * 2.0 ** 9).astype(np.int64)  # exact; rint = ties to even
    out = np.where(sub, ms, out)  # ms == 8 is code 0x08, the smallest normal: same bits
    nor = ~nan & ~sub
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(nor, a, 1.0))).astype(np.int64)
        # guard the log2 rounding at exact powers of two
        e = np.where(np.where(nor, a, 1.0) < np.exp2(e.astype(np.float64)), e - 1, e)
        e = np.where(np.where(nor, a, 1.0) >= np.exp2(e + 1.0), e + 1, e)
        frac = np.where(nor, a, 1.0) / np.exp2(e.astype(np.float64))  # in [1, 2), exact
    mn = np.rint((frac - 1.0) * 8.0).astype(np.int64)
    e = np.where(mn == 8, e + 1, e)
    mn = np.where(mn == 8, 0, mn)
    out = np.where(nor, ((e + 7) << 3) | mn, out)
    out = np.where(nan, E4M3_NAN, out)
    return (out | sign).astype(np.uint8)


def e4m3_step(value) -> np.ndarray:
    """Distance from |value| to the next larger E4M3 magnitude (the format's ulp there)."""
    a = np.abs(np.asarray(value, np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.exp2(e - 3.0)


# ---------------------------------------------------------------- per-row quantisation
TINY_ROW = np.float32(E4M3_MAX * 2.0**-126)  # rows below this amax are stored as zero


def quantize_rows(x_f32):
    """Rows [..., 256] of FP32 values -> (codes uint8 [..., 256], scale f32 [...])."""
    x = np.asarray(x_f32, np.float32)
    amax = np.max(np.abs(x), axis=-1)
    zero = amax < TINY_ROW
    safe = np.where(zero, np.float32(1.0), amax)
    inv = np.float32(E4M3_MAX) / safe  # FP32 division, correctly rounded
    scale = np.where(zero, np.float32(0.0), amax / np.float32(E4M3_MAX)).astype(np.float32)
    y = (x * inv[..., None]).astype(np.float32)  # FP32 product
    codes = np.where(zero[..., None], np.uint8(0), e4m3_encode(y))
    return codes.astype(np.uint8), scale


def dequantize(codes, scale) -> np.ndarray:
    """Exact float64 value of stored rows: code value times the row's scale."""
    return e4m3_decode(codes) * np.asarray(scale, np.float64)[..., None]


# ---------------------------------------------------------------- FP8 layer state
@dataclass
class LayerStateFP8:
    """One layer's state with FP8 rows; metadata as in ``rma_ref.LayerState``."""

    win_k: np.ndarray  # uint8 [B][G][W][D]
    win_v: np.ndarray
    bank_k: np.ndarray
    bank_v: np.ndarray
    pend_k: np.ndarray
    pend_v: np.ndarray
    win_ks: np.ndarray  # f32 [B][G][W]
    win_vs: np.ndarray
    bank_ks: np.ndarray
    bank_vs: np.ndarray
    pend_ks: np.ndarray
    pend_vs: np.ndarray
    bank_score: np.ndarray
    bank_src: np.ndarray
    pend_score: np.ndarray
    pend_src: np.ndarray
    n_bank: np.ndarray
    n_pend: np.ndarray
    pos: np.ndarray

    def copy(self) -> "LayerStateFP8":
        return LayerStateFP8(**{k: np.array(v, copy=True) for k, v in self.__dict__.items()})


def new_layer_state_fp8(batch: int, window: int = R.WINDOW, bank: int = R.BANK,
                        block: int = R.BLOCK, groups: int = R.KV_GROUPS,
                        head_dim: int = R.HEAD_DIM) -> LayerStateFP8:
    c = lambda n: np.zeros((batch, groups, n, head_dim), np.uint8)  # noqa: E731
    s = lambda n: np.zeros((batch, groups, n), np.float32)  # noqa: E731
    return LayerStateFP8(
        win_k=c(window), win_v=c(window), bank_k=c(bank), bank_v=c(bank), pend_k=c(block),
        pend_v=c(block), win_ks=s(window), win_vs=s(window), bank_ks=s(bank), bank_vs=s(bank),
        pend_ks=s(block), pend_vs=s(block),
        bank_score=np.zeros((batch, groups, bank), np.float32),
        bank_src=np.zeros((batch, groups, bank), np.int32),
        pend_score=np.zeros((batch, block, groups), np.float32),
        pend_src=np.zeros((batch, block), np.int32),
        n_bank=np.zeros(batch, np.int32), n_pend=np.zeros(batch, np.int32),
        pos=np.full(batch, -1, np.int32),
    )


def append(st: LayerStateFP8, k_win, v_win, k_rma, v_rma, gk_win, gk_rma, eps: float,
           base: float, score=None, quant=None) -> None:
    """``rma_ref.append`` with each written row quantised (keys from their FP32
    normalised and rotated value, values from their BF16 input).  ``quant`` is the
    row codec (FP32 rows -> codes, scales); E4M3 unless another 8-bit format's is
    given (``oracle.int8_ref``)."""
    quantize_rows_ = quant or quantize_rows
    B = st.pos.shape[0]
    window, block = st.win_k.shape[2], st.pend_k.shape[2]
    for b in range(B):
        p = int(st.pos[b]) + 1
        t = int(st.n_pend[b])
        assert t < block, "pending block is full: commit before appending"
        slot = p % window
        for g in range(st.win_k.shape[1]):
            kw = R.rope(R.rms_norm(R.bf16_to_f64(k_win[b, g]), gk_win, eps), p, base)
            kr = R.rope(R.rms_norm(R.bf16_to_f64(k_rma[b, g]), gk_rma, eps), p, base)
            st.win_k[b, g, slot], st.win_ks[b, g, slot] = quantize_rows_(kw.astype(np.float32))
            st.win_v[b, g, slot], st.win_vs[b, g, slot] = quantize_rows_(
                R.bf16_to_f64(v_win[b, g]).astype(np.float32))
            st.pend_k[b, g, t], st.pend_ks[b, g, t] = quantize_rows_(kr.astype(np.float32))
            st.pend_v[b, g, t], st.pend_vs[b, g, t] = quantize_rows_(
                R.bf16_to_f64(v_rma[b, g]).astype(np.float32))
        st.pend_src[b, t] = p
        if score is not None:
            st.pend_score[b, t, :] = np.asarray(score, np.float32)[b]
        st.n_pend[b] = t + 1
        st.pos[b] = p


def _branch_rows(st: LayerStateFP8, b: int, g: int, branch: str, dequantize=dequantize):
    if branch == "win":
        n = min(int(st.pos[b]) + 1, st.win_k.shape[2])
        return dequantize(st.win_k[b, g, :n], st.win_ks[b, g, :n]), dequantize(
            st.win_v[b, g, :n], st.win_vs[b, g, :n])
    nb, npd = int(st.n_bank[b]), int(st.n_pend[b])
    k = np.concatenate([dequantize(st.bank_k[b, g, :nb], st.bank_ks[b, g, :nb]),
                        dequantize(st.pend_k[b, g, :npd], st.pend_ks[b, g, :npd])])
    v = np.concatenate([dequantize(st.bank_v[b, g, :nb], st.bank_vs[b, g, :nb]),
                        dequantize(st.pend_v[b, g, :npd], st.pend_vs[b, g, :npd])])
    return k, v


def decode_one(keys_by_group, vals_by_group, q_bits, gamma_q, pos: int, eps: float,
               base: float):
    """``rma_ref.decode_one`` over dequantised float64 rows."""
    H = q_bits.shape[0]
    G = len(keys_by_group)
    per = H // G
    o = np.zeros((H, q_bits.shape[1]))
    lse = np.zeros(H)
    for g in range(G):
        for h in range(g * per, (g + 1) * per):
            qh = R.rope(R.rms_norm(R.bf16_to_f64(q_bits[h]), gamma_q, eps), pos, base)
            oh, lh = R.attend(qh[None, :], keys_by_group[g], vals_by_group[g])
            o[h], lse[h] = oh[0], lh[0]
    return o, lse


def decode(st: LayerStateFP8, q_win, q_rma, gq_win, gq_rma, eps: float, base: float,
           deq=None):
    """Both branches for every sequence, as ``rma_ref.decode`` (float64 results).
    ``deq`` is the row decoder (codes, scales -> float64); E4M3 unless given."""
    deq = deq or dequantize
    B = st.pos.shape[0]
    G = st.win_k.shape[1]
    out = {}
    for branch, q, gq in (("win", q_win, gq_win), ("rma", q_rma, gq_rma)):
        o = np.zeros((B, R.Q_HEADS, R.HEAD_DIM))
        lse = np.zeros((B, R.Q_HEADS))
        for b in range(B):
            kv = [_branch_rows(st, b, g, branch, deq) for g in range(G)]
            o[b], lse[b] = decode_one([k for k, _ in kv], [v for _, v in kv], q[b], gq,
                                      int(st.pos[b]), eps, base)
        out[branch] = (o, lse)
    return out["win"][0], out["win"][1], out["rma"][0], out["rma"][1]


def commit(st: LayerStateFP8) -> np.ndarray:
    """``rma_ref.commit``: the same selection and slot rule; admitted rows move with
    their codes and scales."""
    B, G, cap = st.bank_k.shape[0], st.bank_k.shape[1], st.bank_k.shape[2]
    keep = np.full((B, G, cap), -1, np.int32)
    for b in range(B):
        nb, npd = int(st.n_bank[b]), int(st.n_pend[b])
        for g in range(G):
            ki, moves = R.commit_segment(st.bank_score[b, g], st.bank_src[b, g], nb,
                                         st.pend_score[b, :, g], st.pend_src[b], npd, cap)
            keep[b, g] = ki
            for t, s in moves:
                st.bank_k[b, g, s] = st.pend_k[b, g, t]
                st.bank_v[b, g, s] = st.pend_v[b, g, t]
                st.bank_ks[b, g, s] = st.pend_ks[b, g, t]
                st.bank_vs[b, g, s] = st.pend_vs[b, g, t]
                st.bank_score[b, g, s] = st.pend_score[b, t, g]
                st.bank_src[b, g, s] = st.pend_src[b, t]
        st.n_bank[b] = min(cap, nb + npd)
        st.n_pend[b] = 0
    return keep


def kv_bytes_per_unit(window=R.WINDOW, bank=R.BANK, block=R.BLOCK, groups=R.KV_GROUPS,
                      d=R.HEAD_DIM) -> int:
    """Bytes of one (sequence, layer) FP8 state read by a decode step: codes + scales."""
    rows = groups * (window + bank + block)
    return 2 * rows * (d + 4)
