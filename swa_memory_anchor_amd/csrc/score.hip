// Retention scorer: scores = (hidden * W1) * W2, FP32, bias-free, 2560 -> 256 -> 4.
//
// fluxbbs.com "EdgeRock-4B 开源：72 MiB 固定 KV，AIME 82.9 分", section "架构：递归、局部
// 窗口与记忆锚点三件套": a separate small network gives every KV group a retention
// priority through a bias-free projection chain 2560 -> 256 -> 4 computed in FP32.
// The pages name no nonlinearity between the stages; the chain is kept as two
// stages so one could be inserted elementwise.
//
// Design.  Stage 1 is a dense FP32 contraction (256 flop per input byte), so it
// runs on v_mfma_f32_32x32x2f32:
//  * one workgroup (4 waves) per 128-row tile and all 256 columns; each wave owns
//    a 64 x 128 block = 2 x 4 accumulators of 32 x 32;
//  * K is walked in stages of 32: BF16 rows are widened (exactly) to FP32 while
//    being staged in LDS (k-major), W1 rows are staged as is; two LDS buffers, the
//    next stage's global loads in flight while the current stage computes;
//  * stage 2 (x W2, 256 -> 4) is fused: the 128 x 256 block of stage-1 results is
//    passed through LDS in two column halves and every output row is summed over
//    its 256 columns in the same fixed order, so identical input rows give
//    bit-identical scores wherever they sit.
#include "rma_device.h"

namespace rma {

constexpr int kRowsWG = 128;
constexpr int kKt = 32;
constexpr int kAStr = kRowsWG + 4;  // A stage: [k][row], floats
constexpr int kBStr = kMid + 4;     // B stage: [k][col], floats
constexpr int kZStr = 129;          // stage-1 block: [row][col], floats (one column half)
constexpr int kStageFloats = kKt * kAStr + kKt * kBStr;
constexpr int kScoreThreads = 256;

struct ScoreParams {
  const uint16_t *hidden;
  int64_t n_rows, ld_hidden;
  const float *w1, *w2;
  float *scores;
  int64_t ld_scores;
};

__global__ __launch_bounds__(kScoreThreads, 1) void score_kernel(ScoreParams a) {
  __shared__ __align__(16) float smem[2 * kStageFloats];
  __shared__ float w2s[kMid * kGroups];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRowsWG;

  for (int i = tid; i < kMid * kGroups; i += kScoreThreads) w2s[i] = a.w2[i];

  // staging roles
  const int am = tid >> 1, ah = tid & 1;        // A: row am, k half ah (16 values)
  const int bk = tid >> 3, bc = (tid & 7) * 32;  // B: k row bk, columns bc..bc+31
  const bool arow_ok = row0 + am < a.n_rows;
  const uint16_t *arow = a.hidden + (arow_ok ? (row0 + am) : 0) * a.ld_hidden + 16 * ah;

  uint4 ha[2];
  float4 wb[8];
  auto load_stage = [&](int kt) {
    if (arow_ok) {
      ha[0] = *reinterpret_cast<const uint4 *>(arow + kt * kKt);
      ha[1] = *reinterpret_cast<const uint4 *>(arow + kt * kKt + 8);
    } else {
      ha[0] = make_uint4(0, 0, 0, 0);
      ha[1] = ha[0];
    }
    const float *wrow = a.w1 + static_cast<size_t>(kt * kKt + bk) * kMid + bc;
#pragma unroll
    for (int j = 0; j < 8; ++j) wb[j] = *reinterpret_cast<const float4 *>(wrow + 4 * j);
  };
  auto store_stage = [&](int buf) {
    float *As = smem + buf * kStageFloats;
    float *Bs = As + kKt * kAStr;
    const uint32_t w[8] = {ha[0].x, ha[0].y, ha[0].z, ha[0].w, ha[1].x, ha[1].y, ha[1].z, ha[1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      As[(16 * ah + 2 * j) * kAStr + am] = bf16_lo(w[j]);
      As[(16 * ah + 2 * j + 1) * kAStr + am] = bf16_hi(w[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<float4 *>(Bs + bk * kBStr + bc + 4 * j) = wb[j];
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[r][c][q] = 0.f;

  constexpr int nkt = kHidden / kKt;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  const int kl = lane >> 5, ml = lane & 31;
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) load_stage(kt + 1);
    const float *As = smem + (kt & 1) * kStageFloats;
    const float *Bs = As + kKt * kAStr;
#pragma unroll 4
    for (int kk = 0; kk < kKt / 2; ++kk) {
      const int k = 2 * kk + kl;
      const float a0 = As[k * kAStr + wr * 64 + ml];
      const float a1 = As[k * kAStr + wr * 64 + 32 + ml];
      float bv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = Bs[k * kBStr + wc * 128 + 32 * c + ml];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[0][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, bv[c], acc[0][c], 0, 0, 0);
        acc[1][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, bv[c], acc[1][c], 0, 0, 0);
      }
    }
    if (kt + 1 < nkt) store_stage((kt + 1) & 1);
    __syncthreads();
  }

  // Stage 2: s[row][g] = sum_{n=0..255} Z[row][n] * W2[n][g], n ascending.
  float *Z = smem;
  const int srow = tid & (kRowsWG - 1);
  const int sg = (tid >> 7) * 2;  // this thread's two groups
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wc == half) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int row = wr * 64 + r * 32 + 8 * (q >> 2) + 4 * kl + (q & 3);
            Z[row * kZStr + 32 * c + ml] = acc[r][c][q];
          }
    }
    __syncthreads();
    const float *zr = Z + srow * kZStr;
    const float *w2h = w2s + half * 128 * kGroups;
    for (int n = 0; n < 128; ++n) {
      const float z = zr[n];
      s0 = fmaf(z, w2h[n * kGroups + sg], s0);
      s1 = fmaf(z, w2h[n * kGroups + sg + 1], s1);
    }
    __syncthreads();
  }
  if (row0 + srow < a.n_rows) {
    float *out = a.scores + (row0 + srow) * a.ld_scores + sg;
    out[0] = s0;
    out[1] = s1;
  }
}

}  // namespace rma

using namespace rma;

extern "C" rma_status rma_score(const uint16_t *hidden, int64_t n_rows, int64_t ld_hidden,
                                const float *w1, const float *w2, float *scores,
                                int64_t ld_scores, void *stream) {
  if (n_rows < 0 || !w1 || !w2) return RMA_E_ARG;
  if (n_rows == 0) return RMA_OK;
  if (!hidden || !scores) return RMA_E_ARG;
  if (ld_hidden < kHidden || ld_scores < kGroups) return RMA_E_ARG;
  if ((ld_hidden % 8) != 0 || (ld_scores % 4) != 0) return RMA_E_ALIGN;
  if ((reinterpret_cast<uintptr_t>(hidden) & 15u) || (reinterpret_cast<uintptr_t>(w1) & 15u) ||
      (reinterpret_cast<uintptr_t>(scores) & 15u))
    return RMA_E_ALIGN;
  const int64_t blocks = (n_rows + kRowsWG - 1) / kRowsWG;
  if (blocks > 0x7fffffff) return RMA_E_ARG;
  ScoreParams p{hidden, n_rows, ld_hidden, w1, w2, scores, ld_scores};
  hipLaunchKernelGGL(score_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kScoreThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  return RMA_OK;
}
