"""Float64 reference of the Gated DeltaNet (GDN) decode step of EdgeRock-4B.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with the
HIP path.

What the pages fix ([FB] fluxbbs.com "EdgeRock-4B 开源：72 MiB 固定 KV，AIME 82.9 分"):
  * 24 of the 32 layers are Gated DeltaNet layers (three before each SWA||RMA
    layer) that compress the history into a fixed-size recurrent matrix
    [FB "架构：递归、局部窗口与记忆锚点三件套"];
  * the linear-attention part has 16 key heads, 32 value heads and a
    convolution kernel of 4 [same section, the configuration values];
  * the recurrent matrices take 24 MiB and the whole recurrent state 25.50 MiB
    per sequence [FB "72 MiB 是怎么算出来的"; FB "常见问题"]; the GDN state is held
    in FP32 at batch 1 and in FP16 otherwise [FB "72 MiB 是怎么算出来的"].

Head widths (a reading; the pages print none): 24 MiB over 24 layers, 32 value
heads and 2-byte entries leaves d_k * d_v = 16384 per head; the other 1.5 MiB of
recurrent state, read as the convolution's last 4 inputs over all 24 layers in
2-byte entries, leaves 8192 = 2 * 16 * d_k + 32 * d_v channels.  The only
solution is d_k = d_v = 128.

The step (a reading: the pages name Gated DeltaNet but print no formula, so this
is the published gated delta rule, with the per-head conventions of its base
model's public implementation):
  1. the token's projected input x (8192 channels: q | k | v) goes through a
     causal depthwise convolution of width 4 over the last four inputs of each
     channel, then SiLU;
  2. q and k are L2-normalised per head (eps 1e-6) and q is scaled by 1/sqrt(128);
     value head h reads key head floor(h / 2);
  3. decay alpha = exp(-exp(A_log) * softplus(a + dt_bias)), write strength
     beta = sigmoid(b), per value head;
  4. with the state S in R^{d_k x d_v}: S <- alpha S; u = beta (v - S^T k);
     S <- S + k u^T; the output is o = S^T q;
  5. the new state is stored in the state precision (FP16 or FP32, rounding to
     nearest even); the convolution inputs are kept as given (BF16).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .rma_ref import bf16_to_f64

K_HEADS = 16
V_HEADS = 32
HEAD_K = 128
HEAD_V = 128
CONV = 4
KEY_DIM = K_HEADS * HEAD_K  # 2048
VALUE_DIM = V_HEADS * HEAD_V  # 4096
CONV_DIM = 2 * KEY_DIM + VALUE_DIM  # 8192
GDN_LAYERS = 24
L2_EPS = 1e-6


# ---------------------------------------------------------------- scalar maps
def silu(x):
    x = np.asarray(x, np.float64)
    return x / (1.0 + np.exp(-x))


def softplus(x):
    """log(1 + e^x), written so that it neither overflows nor loses small values."""
    x = np.asarray(x, np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """1 / (1 + e^-x), with e^x / (1 + e^x) for negative x so small values keep
    their relative accuracy."""
    x = np.asarray(x, np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def l2_normalize(x, eps: float = L2_EPS):
    """x / sqrt(sum x^2 + eps) over the last axis."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


# ---------------------------------------------------------------- the two state parts
def conv_step(ring, x_new, weight, pos: int):
    """Causal depthwise convolution for the token at position `pos`.

    ring: [4][C] the inputs of positions pos-4..pos-1 in slots (position mod 4)
    (zeros before the stream starts); x_new: [C]; weight: [C][4], tap j
    multiplying the input of position pos-3+j.  Returns (SiLU(conv) [C], the ring
    with x_new in slot pos mod 4)."""
    ring = np.array(ring, np.float64, copy=True)
    x_new = np.asarray(x_new, np.float64)
    w = np.asarray(weight, np.float64)
    ring[pos % CONV] = x_new
    acc = np.zeros(x_new.shape)
    for j in range(CONV):
        acc += w[:, j] * ring[(pos - (CONV - 1) + j) % CONV]
    return silu(acc), ring


def delta_rule_step(S, q, k, v, alpha: float, beta: float):
    """One step of the gated delta rule on one head: S [d_k][d_v], q, k [d_k], v [d_v]
    (q, k already normalised, q scaled).  Returns (new S, o)."""
    S = np.asarray(S, np.float64) * alpha
    k = np.asarray(k, np.float64)
    u = beta * (np.asarray(v, np.float64) - S.T @ k)
    S = S + np.outer(k, u)
    return S, S.T @ np.asarray(q, np.float64)


def gates(a, b, a_log, dt_bias):
    """Per value head: alpha = exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b)."""
    g = -np.exp(np.asarray(a_log, np.float64)) * softplus(np.asarray(a, np.float64) +
                                                           np.asarray(dt_bias, np.float64))
    return np.exp(g), sigmoid(b)


def round_state(S, dtype: str):
    """Store in the state precision: 'f16' (nearest even) or 'f32'."""
    return np.asarray(S, np.float64).astype(np.float16 if dtype == "f16" else np.float32)


# ---------------------------------------------------------------- layer state
@dataclass
class GdnState:
    """One GDN layer for B sequences."""

    S: np.ndarray  # [B][32][128][128], float16 or float32 (the stored precision)
    conv: np.ndarray  # [B][4][8192] uint16 BF16 bits, slot = position mod 4

    def copy(self) -> "GdnState":
        return GdnState(self.S.copy(), self.conv.copy())


def new_state(batch: int, dtype: str = "f16") -> GdnState:
    return GdnState(np.zeros((batch, V_HEADS, HEAD_K, HEAD_V),
                             np.float16 if dtype == "f16" else np.float32),
                    np.zeros((batch, CONV, CONV_DIM), np.uint16))


def split_heads(y):
    """[8192] -> q [16][128], k [16][128], v [32][128] (channel order q | k | v)."""
    return (y[:KEY_DIM].reshape(K_HEADS, HEAD_K), y[KEY_DIM:2 * KEY_DIM].reshape(K_HEADS, HEAD_K),
            y[2 * KEY_DIM:].reshape(V_HEADS, HEAD_V))


def decode_step(st: GdnState, x_bits, a, b, conv_w, a_log, dt_bias, pos, heads=None):
    """One token for every sequence: updates st in place and returns o [B][32][128]
    (float64).  x_bits: [B][8192] BF16 bits (the projected input before the
    convolution); a, b: [B][32]; pos: [B] the token's positions.  `heads` limits the
    recurrence to some value heads (the convolution ring is always updated)."""
    B = x_bits.shape[0]
    dtype = "f16" if st.S.dtype == np.float16 else "f32"
    out = np.zeros((B, V_HEADS, HEAD_V))
    alpha, beta = gates(a, b, a_log, dt_bias)
    for s in range(B):
        p = int(pos[s])
        y, ring = conv_step(bf16_to_f64(st.conv[s]), bf16_to_f64(x_bits[s]), conv_w, p)
        st.conv[s, p % CONV] = x_bits[s]
        q, k, v = split_heads(y)
        qn = l2_normalize(q) / math.sqrt(HEAD_K)
        kn = l2_normalize(k)
        for h in (range(V_HEADS) if heads is None else heads):
            kh = h // (V_HEADS // K_HEADS)
            S_new, o = delta_rule_step(st.S[s, h], qn[kh], kn[kh], v[h], alpha[s, h], beta[s, h])
            st.S[s, h] = round_state(S_new, dtype)
            out[s, h] = o
    return out


def state_bytes_per_sequence(layers: int = GDN_LAYERS, state_bytes: int = 2) -> int:
    """Recurrent matrices plus convolution inputs of one sequence (all GDN layers)."""
    return layers * (V_HEADS * HEAD_K * HEAD_V * state_bytes + CONV * CONV_DIM * 2)


def step_bytes_per_unit(state_bytes: int = 2) -> int:
    """Algorithmic HBM bytes of one (sequence, layer) decode step: the state read and
    written once, three old convolution inputs read and the new one read and stored,
    the gate inputs read and the output written."""
    matrix = V_HEADS * HEAD_K * HEAD_V * state_bytes
    return 2 * matrix + 3 * CONV_DIM * 2 + 2 * CONV_DIM * 2 + 2 * V_HEADS * 4 + V_HEADS * HEAD_V * 2
