// Append one token per sequence to the window ring and the pending block.
//
// neodrop.ai repost of the QbitAI article "内存还会跌吗？KV Cache砍掉99%…", section
// "三段记忆，只记值得记的": the writer emits one candidate record per token.
// fluxbbs.com "EdgeRock-4B 开源：72 MiB 固定 KV…", section "架构：递归、局部窗口与记忆锚点
// 三件套": keys get learned RMS norm and rotary on dims 0..63 (base 1e7); values
// are stored raw.  Keys are finalised here, once, at their own position.
//
// One workgroup per sequence, one wave per KV group, lane l owns dims 4l..4l+3.
#include "rma_device.h"

namespace rma {

struct AppendParams {
  uint16_t *win_k, *win_v, *pend_k, *pend_v;
  float *pend_score;
  int32_t *pend_src, *n_pend, *pos;
  const uint16_t *k_win, *v_win, *k_rma, *v_rma;
  const float *score;
  const float *gk_win, *gk_rma;
  float eps;
  double rope_ratio;  // base^(-1/32)
};

__global__ __launch_bounds__(256) void append_kernel(AppendParams a) {
  const int b = blockIdx.x;
  const int g = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int p = a.pos[b] + 1;
  const int t = a.n_pend[b];
  if (t < 0 || t >= kBlock) return;  // full (or corrupt) pending block: leave untouched
  const int slot = p & (kWindow - 1);
  const size_t in = (static_cast<size_t>(b) * kGroups + g) * kDim + 4 * lane;
  const size_t w_row = ((static_cast<size_t>(b) * kGroups + g) * kWindow + slot) * kDim + 4 * lane;
  const size_t p_row = ((static_cast<size_t>(b) * kGroups + g) * kBlock + t) * kDim + 4 * lane;

  const uint2 kw = *reinterpret_cast<const uint2 *>(a.k_win + in);
  const uint2 kr = *reinterpret_cast<const uint2 *>(a.k_rma + in);
  float xw[4] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y)};
  float xr[4] = {bf16_lo(kr.x), bf16_hi(kr.x), bf16_lo(kr.y), bf16_hi(kr.y)};
  float c, sn;
  rope_cos_sin(a.rope_ratio, p, lane, c, sn);
  norm_rope_head(xw, a.gk_win, a.eps, c, sn, lane);
  norm_rope_head(xr, a.gk_rma, a.eps, c, sn, lane);
  *reinterpret_cast<uint2 *>(a.win_k + w_row) =
      make_uint2(pack_bf16x2(xw[0], xw[1]), pack_bf16x2(xw[2], xw[3]));
  *reinterpret_cast<uint2 *>(a.pend_k + p_row) =
      make_uint2(pack_bf16x2(xr[0], xr[1]), pack_bf16x2(xr[2], xr[3]));
  *reinterpret_cast<uint2 *>(a.win_v + w_row) = *reinterpret_cast<const uint2 *>(a.v_win + in);
  *reinterpret_cast<uint2 *>(a.pend_v + p_row) = *reinterpret_cast<const uint2 *>(a.v_rma + in);
  if (a.score && lane == 0)
    a.pend_score[(static_cast<size_t>(b) * kBlock + t) * kGroups + g] = a.score[b * kGroups + g];
  __syncthreads();  // every wave has read n_pend / pos
  if (threadIdx.x == 0) {
    a.pend_src[static_cast<size_t>(b) * kBlock + t] = p;
    a.n_pend[b] = t + 1;
    a.pos[b] = p;
  }
}

// ---------------------------------------------------------------- FP8 state variant
// Each written row becomes 256 E4M3 codes and one FP32 scale: amax = max |x| over
// the row (a wave reduction), code = E4M3(x * (448 / amax)) with round to nearest
// even (v_cvt_pk_fp8_f32), scale = amax / 448; a row whose amax is below
// 448 * 2^-126 (where 448 / amax would pass 2^126 and the scale would leave the
// normal FP32 range), the all-zero row included, gets zero codes and scale 0.  Keys
// are quantised from their FP32 normalised and rotated value.
struct AppendFp8Params {
  uint8_t *win_k, *win_v, *pend_k, *pend_v;
  float *win_ks, *win_vs, *pend_ks, *pend_vs;
  float *pend_score;
  int32_t *pend_src, *n_pend, *pos;
  const uint16_t *k_win, *v_win, *k_rma, *v_rma;
  const float *score;
  const float *gk_win, *gk_rma;
  float eps;
  double rope_ratio;  // base^(-1/32)
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Quantise one 256-wide row held by a wave (lane l: x[0..3] = dims 4l..4l+3): the
// lane's four codes (one word, dim 4l in the low byte) and the row's scale.
__device__ __forceinline__ uint32_t quantize_row_e4m3(const float x[4], float &scale) {
  const float amax =
      wave_max(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
  constexpr float kTinyRow = 448.0f * 0x1p-126f;
  const bool tiny = amax < kTinyRow;
  const float inv = tiny ? 0.f : 448.0f / amax;
  scale = tiny ? 0.f : amax / 448.0f;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] * inv, x[1] * inv, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] * inv, x[3] * inv, w, true);
  // a tiny or all-zero row stores +0 codes, also where its elements are -0
  return tiny ? 0u : static_cast<uint32_t>(w);
}

// INT8 rows (the same layout): code = round-half-even(x * (127 / amax)) as a signed
// byte, scale = amax / 127; a row whose amax is below 127 * 2^-126 gets zero codes
// and scale 0.  |x * inv| <= 127 up to the rounding of inv and of the product, which
// cannot carry it past 127.5, so no code leaves [-127, 127].
__device__ __forceinline__ uint32_t quantize_row_i8(const float x[4], float &scale) {
  const float amax =
      wave_max(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
  constexpr float kTinyRow = 127.0f * 0x1p-126f;
  const bool tiny = amax < kTinyRow;
  const float inv = tiny ? 0.f : 127.0f / amax;
  scale = tiny ? 0.f : amax / 127.0f;
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int q = static_cast<int>(__builtin_rintf(x[e] * inv));  // ties to even
    w |= (static_cast<uint32_t>(q) & 0xffu) << (8 * e);
  }
  return tiny ? 0u : w;
}

// The 8-bit append for either row codec (E4M3 or INT8).
template <bool kInt8>
__global__ __launch_bounds__(256) void append_q8_kernel(AppendFp8Params a) {
  const int b = blockIdx.x;
  const int g = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int p = a.pos[b] + 1;
  const int t = a.n_pend[b];
  if (t < 0 || t >= kBlock) return;  // full (or corrupt) pending block: leave untouched
  const int slot = p & (kWindow - 1);
  const size_t in = (static_cast<size_t>(b) * kGroups + g) * kDim + 4 * lane;
  const size_t w_row = (static_cast<size_t>(b) * kGroups + g) * kWindow + slot;
  const size_t p_row = (static_cast<size_t>(b) * kGroups + g) * kBlock + t;

  const uint2 kw = *reinterpret_cast<const uint2 *>(a.k_win + in);
  const uint2 kr = *reinterpret_cast<const uint2 *>(a.k_rma + in);
  const uint2 vw = *reinterpret_cast<const uint2 *>(a.v_win + in);
  const uint2 vr = *reinterpret_cast<const uint2 *>(a.v_rma + in);
  float xw[4] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y)};
  float xr[4] = {bf16_lo(kr.x), bf16_hi(kr.x), bf16_lo(kr.y), bf16_hi(kr.y)};
  const float yw[4] = {bf16_lo(vw.x), bf16_hi(vw.x), bf16_lo(vw.y), bf16_hi(vw.y)};
  const float yr[4] = {bf16_lo(vr.x), bf16_hi(vr.x), bf16_lo(vr.y), bf16_hi(vr.y)};
  float c, sn;
  rope_cos_sin(a.rope_ratio, p, lane, c, sn);
  norm_rope_head(xw, a.gk_win, a.eps, c, sn, lane);
  norm_rope_head(xr, a.gk_rma, a.eps, c, sn, lane);
  float s0, s1, s2, s3;
  const uint32_t c0 = kInt8 ? quantize_row_i8(xw, s0) : quantize_row_e4m3(xw, s0);
  const uint32_t c1 = kInt8 ? quantize_row_i8(yw, s1) : quantize_row_e4m3(yw, s1);
  const uint32_t c2 = kInt8 ? quantize_row_i8(xr, s2) : quantize_row_e4m3(xr, s2);
  const uint32_t c3 = kInt8 ? quantize_row_i8(yr, s3) : quantize_row_e4m3(yr, s3);
  *reinterpret_cast<uint32_t *>(a.win_k + w_row * kDim + 4 * lane) = c0;
  *reinterpret_cast<uint32_t *>(a.win_v + w_row * kDim + 4 * lane) = c1;
  *reinterpret_cast<uint32_t *>(a.pend_k + p_row * kDim + 4 * lane) = c2;
  *reinterpret_cast<uint32_t *>(a.pend_v + p_row * kDim + 4 * lane) = c3;
  if (lane == 0) {
    a.win_ks[w_row] = s0;
    a.win_vs[w_row] = s1;
    a.pend_ks[p_row] = s2;
    a.pend_vs[p_row] = s3;
    if (a.score)
      a.pend_score[(static_cast<size_t>(b) * kBlock + t) * kGroups + g] = a.score[b * kGroups + g];
  }
  __syncthreads();  // every wave has read n_pend / pos
  if (threadIdx.x == 0) {
    a.pend_src[static_cast<size_t>(b) * kBlock + t] = p;
    a.n_pend[b] = t + 1;
    a.pos[b] = p;
  }
}

}  // namespace rma

using namespace rma;

static bool aligned8(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

extern "C" rma_status swa_rma_append(const rma_layer_state *st, int32_t batch,
                                     const uint16_t *k_win, const uint16_t *v_win,
                                     const uint16_t *k_rma, const uint16_t *v_rma,
                                     const float *score, const rma_norm *norm, void *stream) {
  if (!st || !norm || !k_win || !v_win || !k_rma || !v_rma) return RMA_E_ARG;
  if (batch <= 0 || batch > RMA_MAX_BATCH) return RMA_E_ARG;
  if (!st->win_k || !st->win_v || !st->pend_k || !st->pend_v || !st->pend_src || !st->n_pend ||
      !st->pos || !norm->gk_win || !norm->gk_rma || (score && !st->pend_score))
    return RMA_E_ARG;
  const void *a16[] = {st->win_k, st->win_v, st->pend_k, st->pend_v, norm->gk_win, norm->gk_rma};
  for (const void *p : a16)
    if (!aligned16(p)) return RMA_E_ALIGN;
  const void *a8[] = {k_win, v_win, k_rma, v_rma};
  for (const void *p : a8)
    if (!aligned8(p)) return RMA_E_ALIGN;
  AppendParams p;
  p.win_k = st->win_k;
  p.win_v = st->win_v;
  p.pend_k = st->pend_k;
  p.pend_v = st->pend_v;
  p.pend_score = st->pend_score;
  p.pend_src = st->pend_src;
  p.n_pend = st->n_pend;
  p.pos = st->pos;
  p.k_win = k_win;
  p.v_win = v_win;
  p.k_rma = k_rma;
  p.v_rma = v_rma;
  p.score = score;
  p.gk_win = norm->gk_win;
  p.gk_rma = norm->gk_rma;
  p.eps = norm->eps;
  p.rope_ratio = rope_ratio(norm->rope_base);
  hipLaunchKernelGGL(append_kernel, dim3(batch), dim3(256), 0, static_cast<hipStream_t>(stream), p);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  return RMA_OK;
}

template <bool kInt8>
static rma_status append_q8(const rma_layer_state_fp8 *st, int32_t batch,
                            const uint16_t *k_win, const uint16_t *v_win,
                            const uint16_t *k_rma, const uint16_t *v_rma, const float *score,
                            const rma_norm *norm, void *stream) {
  if (!st || !norm || !k_win || !v_win || !k_rma || !v_rma) return RMA_E_ARG;
  if (batch <= 0 || batch > RMA_MAX_BATCH) return RMA_E_ARG;
  if (!st->win_k || !st->win_v || !st->pend_k || !st->pend_v || !st->win_ks || !st->win_vs ||
      !st->pend_ks || !st->pend_vs || !st->pend_src || !st->n_pend || !st->pos ||
      !norm->gk_win || !norm->gk_rma || (score && !st->pend_score))
    return RMA_E_ARG;
  const void *a16[] = {st->win_k,  st->win_v,  st->pend_k,  st->pend_v,   st->win_ks,
                       st->win_vs, st->pend_ks, st->pend_vs, norm->gk_win, norm->gk_rma};
  for (const void *p : a16)
    if (!aligned16(p)) return RMA_E_ALIGN;
  const void *a8[] = {k_win, v_win, k_rma, v_rma};
  for (const void *p : a8)
    if (!aligned8(p)) return RMA_E_ALIGN;
  AppendFp8Params p;
  p.win_k = st->win_k;
  p.win_v = st->win_v;
  p.pend_k = st->pend_k;
  p.pend_v = st->pend_v;
  p.win_ks = st->win_ks;
  p.win_vs = st->win_vs;
  p.pend_ks = st->pend_ks;
  p.pend_vs = st->pend_vs;
  p.pend_score = st->pend_score;
  p.pend_src = st->pend_src;
  p.n_pend = st->n_pend;
  p.pos = st->pos;
  p.k_win = k_win;
  p.v_win = v_win;
  p.k_rma = k_rma;
  p.v_rma = v_rma;
  p.score = score;
  p.gk_win = norm->gk_win;
  p.gk_rma = norm->gk_rma;
  p.eps = norm->eps;
  p.rope_ratio = rope_ratio(norm->rope_base);
  hipLaunchKernelGGL(append_q8_kernel<kInt8>, dim3(batch), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  return RMA_OK;
}

extern "C" rma_status swa_rma_append_fp8(const rma_layer_state_fp8 *st, int32_t batch,
                                         const uint16_t *k_win, const uint16_t *v_win,
                                         const uint16_t *k_rma, const uint16_t *v_rma,
                                         const float *score, const rma_norm *norm, void *stream) {
  return append_q8<false>(st, batch, k_win, v_win, k_rma, v_rma, score, norm, stream);
}

extern "C" rma_status swa_rma_append_i8(const rma_layer_state_fp8 *st, int32_t batch,
                                        const uint16_t *k_win, const uint16_t *v_win,
                                        const uint16_t *k_rma, const uint16_t *v_rma,
                                        const float *score, const rma_norm *norm, void *stream) {
  return append_q8<true>(st, batch, k_win, v_win, k_rma, v_rma, score, norm, stream);
}
