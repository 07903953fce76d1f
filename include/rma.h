/*
 * rma.h - C ABI of the Rock Memory Anchors (RMA) hot path for AMD MI355X (gfx950).
 *
 * What is computed follows the pages about EdgeRock-4B:
 *   [FB]  fluxbbs.com, "EdgeRock-4B 开源：72 MiB 固定 KV，AIME 82.9 分",
 *         section "72 MiB 是怎么算出来的" (the five bounded state parts and their
 *         sizes: window, committed bank, pending block, all BF16) and section
 *         "架构：递归、局部窗口与记忆锚点三件套" (SWA 1024 in parallel with RMA; the
 *         FP32 bias-free 2560->256->4 scorer; per-group selection; 16 query heads
 *         over 4 KV groups, head width 256; learned RMS norm on q and k; rotary
 *         on 64 of 256 dims with base 1e7; values neither rotated nor normed;
 *         1024 committed + 256 candidates per group).
 *   [QB]  neodrop.ai repost of the QbitAI article "内存还会跌吗？KV Cache砍掉99%…",
 *         section "三段记忆，只记值得记的" (one candidate record per token; every 256
 *         candidates are ranked together with the bank and the best 1024 kept,
 *         each KV group on its own; kept anchors never change).
 *
 * Readings where the pages leave a step open:
 *   - RMS norm y = x / sqrt(mean(x^2) + eps) * gamma over one head (eps is a
 *     runtime value, 1e-6 by default); one gain vector per branch and role.
 *   - Rotary pairs (i, i+32) inside dims 0..63, theta_i = base^(-2i/64).
 *   - Keys are normalised and rotated once when appended, at their own
 *     position; queries at the current position on every read.
 *   - Head h reads KV group h/4; softmax scale 1/16.
 *   - The anchor branch reads bank slots [0, n_bank) then pending slots
 *     [0, n_pend) under one softmax.  Both branches are returned with their
 *     natural-log log-sum-exps; how they are combined is the caller's choice.
 *   - Ties in score keep the lower source position; -0.0 equals +0.0; NaN
 *     ranks below every number.
 *
 * Conventions (all entry points):
 *   - Every pointer is caller-owned device memory unless stated otherwise.
 *     The library allocates nothing.  Its only mutable global state is the
 *     per-GPU array of swa_rma_decode_attn_noalloc (see there).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream) and never synchronises the host.
 *   - The return value reports host-detectable errors only: bad arguments,
 *     misalignment (K/V, hidden and query rows must be 16-byte aligned),
 *     undersized workspace, or a launch error.  Nothing is launched when a
 *     check fails.
 *   - Device-side contract (not checked on the host): 0 <= n_bank <= 1024,
 *     0 <= n_pend <= 256, n_pend < 256 before an append, and distinct,
 *     non-negative source positions within a group.  Kernels clamp counts to their capacities so
 *     that no access leaves the arrays.
 */
#ifndef RMA_H
#define RMA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Geometry (compile-time; [FB] both sections above, [QB] section above). */
#define RMA_Q_HEADS 16
#define RMA_KV_GROUPS 4
#define RMA_HEAD_DIM 256
#define RMA_ROPE_DIM 64
#define RMA_WINDOW 1024
#define RMA_BANK 1024
#define RMA_BLOCK 256
#define RMA_HIDDEN 2560
#define RMA_SCORER_MID 256
#define RMA_MAX_BATCH 65536
#define RMA_MAX_JOBS 16 /* calls one *_multi entry point takes at most */

typedef enum {
  RMA_OK = 0,
  RMA_E_ARG = 1,       /* null pointer, batch out of range, bad stride */
  RMA_E_ALIGN = 2,     /* a row pointer or stride breaks 16-byte alignment */
  RMA_E_WORKSPACE = 3, /* workspace missing or smaller than the entry point needs */
  RMA_E_HIP = 4        /* the HIP runtime reported an error at launch */
} rma_status;

/*
 * One SWA||RMA layer's attention state for `batch` sequences ([FB] section
 * "72 MiB 是怎么算出来的").  All arrays are row-major, dense, in device memory.
 *   win_k, win_v   bf16 [B][4][1024][256]  ring slot = position mod 1024; keys
 *                                          stored normalised and rotated.
 *   bank_k, bank_v bf16 [B][4][1024][256]  slots [0, n_bank) valid (a prefix).
 *   bank_score     f32  [B][4][1024]       retention priority of each bank record.
 *   bank_src       i32  [B][4][1024]       source position of each bank record.
 *   pend_k, pend_v bf16 [B][4][256][256]   slots [0, n_pend) valid.
 *   pend_score     f32  [B][256][4]        row = pending token, column = KV group
 *                                          (the layout rma_score writes).
 *   pend_src       i32  [B][256]           one source position per pending token.
 *   n_bank, n_pend i32  [B]
 *   pos            i32  [B]                newest appended position, -1 = none.
 * BF16 values are passed as their 16-bit patterns.
 */
typedef struct rma_layer_state {
  uint16_t *win_k, *win_v;
  uint16_t *bank_k, *bank_v;
  float *bank_score;
  int32_t *bank_src;
  uint16_t *pend_k, *pend_v;
  float *pend_score;
  int32_t *pend_src;
  int32_t *n_bank, *n_pend;
  int32_t *pos;
} rma_layer_state;

/* Learned RMS-norm gains (f32 [256] each, device memory) and scalars. */
typedef struct rma_norm {
  const float *gq_win, *gk_win, *gq_rma, *gk_rma;
  float eps;       /* RMS norm epsilon (1e-6) */
  float rope_base; /* rotary base (1e7) */
} rma_norm;

/* Bytes of all arrays of one layer's state for `batch` sequences (closed form,
 * host only): K/V (9 MiB per sequence) plus scores, sources and counters. */
size_t rma_layer_state_bytes(int32_t batch);

/* K/V bytes alone: batch * 2 * 4 * (1024 + 1024 + 256) * 256 * 2 = batch * 9 MiB
 * per layer; eight layers give the 72 MiB per sequence of [FB]. */
size_t rma_layer_kv_bytes(int32_t batch);

/* Workspace that swa_rma_decode_attn needs at this batch (0 when none). */
size_t rma_decode_workspace_bytes(int32_t batch);

/* Number of key-range splits swa_rma_decode_attn uses at this batch. */
int32_t rma_decode_splits(int32_t batch);

/*
 * swa_rma_append - write the next token of every sequence ([QB] section above:
 * one candidate per token; [FB] section "架构…": q/k norms, partial rotary).
 *   k_win, v_win, k_rma, v_rma  bf16 [B][4][256], raw (before norm/rotary).
 *   score   f32 [B][4] written to pend_score[b][n_pend][:], or NULL to leave
 *           the row for a later rma_score burst.
 * For each sequence b with p = pos[b] + 1 and t = n_pend[b]:
 *   win_k[b][g][p % 1024] = bf16(rope_p(rmsnorm(k_win[b][g]) * gk_win));
 *   win_v[b][g][p % 1024] = v_win[b][g];
 *   pend_k[b][g][t]       = bf16(rope_p(rmsnorm(k_rma[b][g]) * gk_rma));
 *   pend_v[b][g][t]       = v_rma[b][g];   pend_src[b][t] = p;
 *   n_pend[b] = t + 1;  pos[b] = p.
 * A sequence whose pending block is already full (t >= 256) is left untouched.
 */
rma_status swa_rma_append(const rma_layer_state *st, int32_t batch, const uint16_t *k_win,
                          const uint16_t *v_win, const uint16_t *k_rma, const uint16_t *v_rma,
                          const float *score, const rma_norm *norm, void *stream);

/*
 * swa_rma_decode_attn - decode-step attention of one SWA||RMA layer ([FB]
 * section "架构…": SWA 1024 in parallel with RMA, 16 q heads / 4 KV groups).
 *   q_win, q_rma  bf16 [B][16][256], raw; they may alias.
 *   o_win, o_rma  bf16 [B][16][256] out: softmax-weighted values.
 *   lse_win, lse_rma f32 [B][16] out: natural-log log-sum-exp of the scaled scores.
 * Window branch: keys in ring slots [0, min(pos+1, 1024)).  Anchor branch:
 * bank slots [0, n_bank) followed by pending slots [0, n_pend).  Query head h
 * is rope_pos(rmsnorm(q[h]) * gq) and reads group h/4 with scale 1/16.  A
 * branch with no keys yields o = 0 and lse = -inf.
 * `workspace` must hold rma_decode_workspace_bytes(batch) bytes (may be NULL
 * when that is 0) and be 16-byte aligned.
 */
rma_status swa_rma_decode_attn(const rma_layer_state *st, int32_t batch, const uint16_t *q_win,
                               const uint16_t *q_rma, const rma_norm *norm, uint16_t *o_win,
                               float *lse_win, uint16_t *o_rma, float *lse_rma, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * swa_rma_decode_attn_noalloc - swa_rma_decode_attn for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (minus the workspace) and the
 * same results, bit for bit.  The split partials go to a device array of the
 * library instead, RMA_NOALLOC_SCRATCH_BYTES per GPU, held until the process
 * ends; that covers every batch (the largest need, at batch 63, is 4,193,280
 * bytes; batches of 64 and more need none).  Nothing is allocated: the first call
 * on a device only looks up the array's device address (hipGetSymbolAddress, with
 * that device made current), so make the first call outside graph capture.
 * All calls on one GPU share the array and nothing in it must start at zero;
 * calls that overlap on one GPU (on different streams or host threads) race and
 * give undefined results.  Returns RMA_E_WORKSPACE if a batch would need more
 * than the array holds, RMA_E_HIP if the address lookup fails.
 */
#define RMA_NOALLOC_SCRATCH_BYTES (4u << 20)
rma_status swa_rma_decode_attn_noalloc(const rma_layer_state *st, int32_t batch,
                                       const uint16_t *q_win, const uint16_t *q_rma,
                                       const rma_norm *norm, uint16_t *o_win, float *lse_win,
                                       uint16_t *o_rma, float *lse_rma, void *stream);

/* Workspace that swa_rma_step needs at this batch: the decode's split partials,
 * then one 32-bit counter per sequence at a 256-byte aligned offset. */
size_t rma_step_workspace_bytes(int32_t batch);

/*
 * swa_rma_step - one token per sequence, appended and attended in one launch
 * (and the split merge where the decode splits): the same state and outputs as
 * swa_rma_append(st, k_win, v_win, k_rma, v_rma, score) followed by
 * swa_rma_decode_attn(st, q_win, q_rma), bit for bit.  Arguments as in those two.
 * The new token's key and value are attended to by its own query.  A sequence
 * whose pending block is full takes no token and attends to the state as it is.
 * `workspace` must hold rma_step_workspace_bytes(batch) bytes, 16-byte aligned,
 * all zero before its first use; every completed call leaves its counters at
 * zero again, so the same workspace serves later calls (and decodes) as it is.
 * Calls that share a workspace must not overlap.
 */
rma_status swa_rma_step(const rma_layer_state *st, int32_t batch, const uint16_t *k_win,
                        const uint16_t *v_win, const uint16_t *k_rma, const uint16_t *v_rma,
                        const float *score, const uint16_t *q_win, const uint16_t *q_rma,
                        const rma_norm *norm, uint16_t *o_win, float *lse_win, uint16_t *o_rma,
                        float *lse_rma, void *workspace, size_t workspace_bytes, void *stream);

/*
 * rma_score - retention priorities ([FB] section "架构…": bias-free FP32 chain
 * 2560 -> 256 -> 4, one priority per KV group).
 *   hidden  bf16 [n_rows][ld_hidden] (first 2560 columns used), ld_hidden a
 *           multiple of 8 and >= 2560.
 *   w1      f32 [2560][256];  w2 f32 [256][4].
 *   scores  f32 [n_rows][ld_scores] out (first 4 columns), ld_scores >= 4, a
 *           multiple of 4.  With ld_scores = 4 and rows ordered (b, token) the
 *           output is exactly pend_score.
 * scores = (hidden * w1) * w2, FP32 arithmetic; identical rows give identical
 * results wherever they sit.  n_rows = 0 is a no-op.
 */
rma_status rma_score(const uint16_t *hidden, int64_t n_rows, int64_t ld_hidden, const float *w1,
                     const float *w2, float *scores, int64_t ld_scores, void *stream);

/* One call of rma_score inside rma_score_multi (device pointers, as in rma_score). */
typedef struct rma_score_job {
  const uint16_t *hidden;
  const float *w1, *w2;
  float *scores;
} rma_score_job;

/*
 * rma_score_multi - n_jobs (1..RMA_MAX_JOBS) independent rma_score calls with the
 * same n_rows, ld_hidden and ld_scores in one launch, e.g. every layer's scores
 * of a block.  `jobs` is a host array; each job's results are those of rma_score
 * with its pointers, bit for bit.  Any job failing the checks of rma_score fails
 * the call and nothing is launched.
 */
rma_status rma_score_multi(const rma_score_job *jobs, int32_t n_jobs, int64_t n_rows,
                           int64_t ld_hidden, int64_t ld_scores, void *stream);

/*
 * rma_score_workspace_bytes - workspace rma_score_multi_ws needs for n_jobs
 * calls of n_rows rows each: n_jobs * n_rows * 1024 bytes (the 256 stage-1
 * results of every row, FP32) when the calls are small enough for its split
 * path (n_jobs * ceil(n_rows / 32) <= 256), else 0.  0 for n_jobs outside
 * 1..RMA_MAX_JOBS.
 */
size_t rma_score_workspace_bytes(int32_t n_jobs, int64_t n_rows);

/*
 * rma_score_multi_ws - rma_score_multi for calls too small to give every CU a
 * row tile (the scores of a 256-token block at batch 1, [QB] section "三段记忆…":
 * candidates are scored once per 256-token block).  Arguments and results as
 * rma_score_multi, bit for bit; in addition
 *   workspace  device memory of rma_score_workspace_bytes(n_jobs, n_rows) bytes,
 *              16-byte aligned, owned by the caller; may be NULL when that size
 *              is 0.  Its contents need no initial value and are scratch after
 *              the call (stage-1 results).  Calls sharing a workspace must not
 *              overlap.
 * Small calls run as two launches: one wave per 32 x 32 block of stage-1 results
 * (the 256 columns of a row tile spread over 8 CUs), then the fixed-order sum of
 * each row over its 256 columns.  Larger calls run rma_score_multi's launch and
 * leave the workspace untouched.
 * Errors: those of rma_score_multi; RMA_E_WORKSPACE when the workspace is NULL or
 * smaller than required, RMA_E_ALIGN when it is not 16-byte aligned (nothing is
 * launched in either case).
 */
rma_status rma_score_multi_ws(const rma_score_job *jobs, int32_t n_jobs, int64_t n_rows,
                              int64_t ld_hidden, int64_t ld_scores, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * rma_commit_topk - commit every sequence's pending block ([QB] section above:
 * each KV group keeps the best 1024 of bank + pending; [FB] section "架构…":
 * groups choose independently and may keep the same positions).
 * Order: higher score first, equal scores keep the lower source position.
 * Slots are stable: survivors stay put; admitted pending rows, in ascending
 * pending order, are copied (K, V, score, source) into the free slots (evicted
 * slots and slots >= n_bank) in ascending slot order.  Then
 * n_bank = min(1024, n_bank + n_pend) and n_pend = 0.
 *   keep_idx  i32 [B][4][1024] out, or NULL: s for a surviving bank record in
 *             slot s, 1024 + t for pending row t written to slot s, -1 if empty.
 */
rma_status rma_commit_topk(const rma_layer_state *st, int32_t batch, int32_t *keep_idx,
                           void *stream);

/*
 * rma_commit_topk_multi - rma_commit_topk on n_states (1..RMA_MAX_JOBS) layer
 * states of the same batch in one launch (plus one launch for the counters), e.g.
 * every layer at a block's end.  `states` is a host array; keep_idx is NULL or a
 * host array of n_states device pointers (each may be NULL).  Each state ends as
 * rma_commit_topk would leave it, bit for bit.
 */
rma_status rma_commit_topk_multi(const rma_layer_state *states, int32_t n_states, int32_t batch,
                                 int32_t *const *keep_idx, void *stream);

/* Workspace that swa_rma_prefill needs for `n_tokens` tokens per sequence. */
size_t rma_prefill_workspace_bytes(int32_t batch, int32_t n_tokens);

/*
 * swa_rma_prefill - chunked prefill of one layer: n_tokens (1..256) tokens per
 * sequence in one call.  The result is that of n_tokens successive
 * swa_rma_append + swa_rma_decode_attn steps ([FB] section "架构…", [QB] section
 * above): token i of sequence b sits at position p = pos[b] + 1 + i and attends
 * to window positions p-1023..p, to all committed anchors and to the pending
 * records at positions <= p.
 *   k_win, v_win, k_rma, v_rma  bf16 [B][n_tokens][4][256], raw.
 *   score   f32 [B][n_tokens][4] into pend_score, or NULL.
 *   q_win, q_rma  bf16 [B][n_tokens][16][256], raw; they may alias.
 *   o_win, o_rma  bf16 [B][n_tokens][16][256] out; lse_win, lse_rma f32
 *                 [B][n_tokens][16] out.
 *   workspace  rma_prefill_workspace_bytes(batch, n_tokens) bytes, 16-byte aligned.
 * The pending block must have room: n_pend[b] + n_tokens <= 256 (commit first);
 * a sequence without room is left untouched and its outputs are o = 0,
 * lse = -inf.  Afterwards n_pend[b] += n_tokens and pos[b] += n_tokens.
 */
rma_status swa_rma_prefill(const rma_layer_state *st, int32_t batch, int32_t n_tokens,
                           const uint16_t *k_win, const uint16_t *v_win, const uint16_t *k_rma,
                           const uint16_t *v_rma, const float *score, const uint16_t *q_win,
                           const uint16_t *q_rma, const rma_norm *norm, uint16_t *o_win,
                           float *lse_win, uint16_t *o_rma, float *lse_rma, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * FP8 state variant.  The pages list quantised releases of the model's weights
 * ([FB] section "架构…"; [QB] section "开源到哪一步") but no format for the
 * attention state; this variant is a reading of this library:
 *   - every stored K and V row (256 values) is 256 OCP FP8 E4M3 codes plus one
 *     FP32 scale = amax / 448 (amax = max |x| over the row, FP32; a row with
 *     amax below 448 * 2^-126, the all-zero row included, has scale 0 and zero
 *     codes);
 *   - code = E4M3(x * (448 / amax)), products and quotient in FP32, E4M3
 *     rounding to nearest, ties to even; the row means code value * scale;
 *   - keys are quantised from their FP32 normalised and rotated value, values
 *     from their BF16 input.
 * Layout: as rma_layer_state with 1-byte codes, plus one scale array per K/V
 * array:
 *   win_k, win_v   u8  [B][4][1024][256]   win_ks, win_vs   f32 [B][4][1024]
 *   bank_k, bank_v u8  [B][4][1024][256]   bank_ks, bank_vs f32 [B][4][1024]
 *   pend_k, pend_v u8  [B][4][256][256]    pend_ks, pend_vs f32 [B][4][256]
 *   bank_score, bank_src, pend_score, pend_src, n_bank, n_pend, pos as above.
 * Code arrays and scale arrays must be 16-byte aligned.  A decode step reads
 * 4,792,320 B of K/V state per sequence and layer, against 9,437,184 in BF16.
 */
typedef struct rma_layer_state_fp8 {
  uint8_t *win_k, *win_v;
  uint8_t *bank_k, *bank_v;
  uint8_t *pend_k, *pend_v;
  float *win_ks, *win_vs;
  float *bank_ks, *bank_vs;
  float *pend_ks, *pend_vs;
  float *bank_score;
  int32_t *bank_src;
  float *pend_score;
  int32_t *pend_src;
  int32_t *n_bank, *n_pend;
  int32_t *pos;
} rma_layer_state_fp8;

/* Bytes of all arrays of one layer's FP8 state for `batch` sequences. */
size_t rma_layer_state_fp8_bytes(int32_t batch);

/* swa_rma_append for the FP8 state: the same rows, quantised as described above. */
rma_status swa_rma_append_fp8(const rma_layer_state_fp8 *st, int32_t batch, const uint16_t *k_win,
                              const uint16_t *v_win, const uint16_t *k_rma, const uint16_t *v_rma,
                              const float *score, const rma_norm *norm, void *stream);

/* swa_rma_decode_attn over the FP8 state: the attention of the dequantised rows
 * (score of a key times its scale; values weighed by their scales).  Same
 * outputs, workspace (rma_decode_workspace_bytes) and error behaviour. */
rma_status swa_rma_decode_attn_fp8(const rma_layer_state_fp8 *st, int32_t batch,
                                   const uint16_t *q_win, const uint16_t *q_rma,
                                   const rma_norm *norm, uint16_t *o_win, float *lse_win,
                                   uint16_t *o_rma, float *lse_rma, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* rma_commit_topk for the FP8 state: the same selection and slot rule; an
 * admitted row moves with its codes and its K and V scales.  The codes are moved
 * as bytes, so the same call commits an INT8 state (below). */
rma_status rma_commit_topk_fp8(const rma_layer_state_fp8 *st, int32_t batch, int32_t *keep_idx,
                               void *stream);

/*
 * INT8 state variant (the pages list INT8 releases beside FP8 ones, [FB] section
 * "架构…", [QB] section "开源到哪一步"; the format is, as for FP8, a reading of this
 * library).  The layout is rma_layer_state_fp8's, and rma_layer_state_fp8_bytes
 * and rma_commit_topk_fp8 serve it as they are; only the meaning of a code
 * differs:
 *   - every stored K and V row is 256 signed 8-bit codes (two's complement) plus
 *     one FP32 scale = amax / 127 (a row with amax below 127 * 2^-126, the
 *     all-zero row included, has scale 0 and zero codes);
 *   - code = round-half-even(x * (127 / amax)), quotient and product in FP32, so
 *     |code| <= 127; the row means code * scale;
 *   - keys are quantised from their FP32 normalised and rotated value, values
 *     from their BF16 input.
 */

/* swa_rma_append for the INT8 state: the same rows, quantised as described above.
 * Arguments, alignment and error behaviour as swa_rma_append_fp8. */
rma_status swa_rma_append_i8(const rma_layer_state_fp8 *st, int32_t batch, const uint16_t *k_win,
                             const uint16_t *v_win, const uint16_t *k_rma, const uint16_t *v_rma,
                             const float *score, const rma_norm *norm, void *stream);

/* swa_rma_decode_attn over the INT8 state: the attention of the dequantised rows.
 * Arguments, outputs, workspace and error behaviour as swa_rma_decode_attn_fp8. */
rma_status swa_rma_decode_attn_i8(const rma_layer_state_fp8 *st, int32_t batch,
                                  const uint16_t *q_win, const uint16_t *q_rma,
                                  const rma_norm *norm, uint16_t *o_win, float *lse_win,
                                  uint16_t *o_rma, float *lse_rma, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Human-readable name of a status code (static string). */
const char *rma_status_str(rma_status s);

#ifdef __cplusplus
}
#endif

#endif /* RMA_H */
