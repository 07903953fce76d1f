/*
 * gdn.h - C ABI of the Gated DeltaNet (GDN) decode step of EdgeRock-4B for AMD
 * MI355X (gfx950): the recurrent layers that sit beside the SWA||RMA layers.
 *
 * What the pages fix ([FB] fluxbbs.com "EdgeRock-4B 开源：72 MiB 固定 KV，AIME 82.9 分"):
 *   - section "架构：递归、局部窗口与记忆锚点三件套": 24 Gated DeltaNet layers compress
 *     the history into a fixed-size recurrent matrix; the linear-attention part
 *     has 16 key heads, 32 value heads and a convolution kernel of 4;
 *   - section "72 MiB 是怎么算出来的": the recurrent matrices take 24 MiB per
 *     sequence and the GDN state is FP32 at batch 1, FP16 otherwise;
 *   - section "常见问题": the recurrent state is 25.50 MiB per sequence in all.
 *
 * Readings where the pages leave a step open:
 *   - head widths d_k = d_v = 128: the unique solution of the two printed sizes
 *     (matrices 24 layers x 32 heads x d_k x d_v x 2 B = 24 MiB; the other 1.5 MiB
 *     the convolution's last 4 inputs of 2 x 16 x d_k + 32 x d_v channels, 2 B each);
 *   - the step is the published gated delta rule with the per-head conventions
 *     of the base model's public implementation: depthwise causal convolution
 *     of width 4 over the q | k | v channels, then SiLU; q and k L2-normalised
 *     per head (eps 1e-6), q scaled by 1/sqrt(128); value head h reads key head
 *     h/2; alpha = exp(-exp(A_log) * softplus(a + dt_bias)), beta = sigmoid(b);
 *     S <- alpha S; u = beta (v - S^T k); S <- S + k u^T; o = S^T q, with
 *     S in R^{128 x 128} (key dim x value dim) per value head.
 *
 * Conventions as in rma.h: caller-owned device memory, nothing allocated, no
 * global state, asynchronous on `stream`, host-detectable errors only.
 */
#ifndef GDN_H
#define GDN_H

#include "rma.h"

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_K_HEADS 16
#define GDN_V_HEADS 32
#define GDN_HEAD_DIM 128  /* key and value head width */
#define GDN_CONV 4        /* convolution width */
#define GDN_CONV_DIM 8192 /* q (16 x 128) | k (16 x 128) | v (32 x 128) channels */

/* Precision of the recurrent matrices: FP16 for batched decoding, FP32 at batch 1. */
#define GDN_STATE_F16 0
#define GDN_STATE_F32 1

/* One GDN layer's state for `batch` sequences (caller-owned, 16-byte aligned). */
typedef struct gdn_layer_state {
  void *S;        /* [B][32][128 key dims][128 value dims], FP16 or FP32 (row-major) */
  uint16_t *conv; /* bf16 [B][4][8192]: the convolution input of position p in slot p mod 4;
                     zero before a stream starts */
} gdn_layer_state;

/* One GDN layer's parameters (device memory, FP32). */
typedef struct gdn_params {
  const float *conv_w;  /* [8192][4]: tap j multiplies the input of position p - 3 + j */
  const float *a_log;   /* [32] */
  const float *dt_bias; /* [32] */
} gdn_params;

/* Bytes of one layer's state (matrices + convolution inputs) for `batch`
 * sequences; 0 for batch <= 0 or an unknown dtype.  Host-only. */
size_t gdn_layer_state_bytes(int32_t batch, int32_t state_dtype);

/*
 * One decode step of one GDN layer for every sequence of the batch:
 *   x       bf16 [B][8192]  the token's projected input (q | k | v channels), before
 *                           the convolution;
 *   a, b    f32  [B][32]    the decay and write-strength inputs per value head;
 *   pos     i32  [B]        the token's position (>= 0; selects the ring slot);
 *   o       bf16 [B][32][128] output, o = S^T q per value head (before the model's
 *                           gated output norm).
 * Updates st->S in place and stores x into ring slot pos mod 4.  Each new matrix
 * element is one FP32 fused multiply-add; FP16 state stores that FP32 value rounded
 * to nearest even.  Errors:
 * RMA_E_ARG (null pointer, batch outside 1..RMA_MAX_BATCH, unknown dtype),
 * RMA_E_ALIGN (S, conv, x, o or conv_w not 16-byte aligned), RMA_E_HIP.
 */
rma_status gdn_decode_step(const gdn_layer_state *st, int32_t batch, int32_t state_dtype,
                           const uint16_t *x, const float *a, const float *b,
                           const int32_t *pos, const gdn_params *prm, uint16_t *o,
                           void *stream);

/* Most tokens one gdn_prefill call takes. */
#define GDN_MAX_PREFILL 65536

/*
 * gdn_prefill - n_tokens (1..GDN_MAX_PREFILL) tokens per sequence through one GDN
 * layer in one call: the result is that of n_tokens successive gdn_decode_step
 * calls with positions pos[b], pos[b] + 1, ..., bit for bit (the matrices are
 * rounded to their storage type after every token, as stored steps would be).
 *   x       bf16 [B][n_tokens][8192]  the tokens' projected inputs;
 *   a, b    f32  [B][n_tokens][32];
 *   pos     i32  [B]  position of each sequence's first token of the chunk (>= 0);
 *   o       bf16 [B][n_tokens][32][128] out.
 * Afterwards the ring holds the inputs of the chunk's last min(n_tokens, 4) tokens
 * (slot = position mod 4; other slots unchanged); the caller advances its
 * positions by n_tokens.  Errors as gdn_decode_step, and RMA_E_ARG for n_tokens
 * out of range.
 */
rma_status gdn_prefill(const gdn_layer_state *st, int32_t batch, int32_t n_tokens,
                       int32_t state_dtype, const uint16_t *x, const float *a, const float *b,
                       const int32_t *pos, const gdn_params *prm, uint16_t *o, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
