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
//  * K is walked in slices of 32: BF16 rows are widened (exactly) to FP32 while
//    being staged in LDS row-major (m-major), W1 is staged column-major (n-major);
//    each lane's 16 operands of a slice are then contiguous, so a slice's operands
//    come in with 24 16-byte LDS reads and its 128 MFMAs issue back to back; two
//    LDS buffers, the next slice's global loads in flight meanwhile;
//  * stage 2 (x W2, 256 -> 4) is fused: the 128 x 256 block of stage-1 results is
//    passed through LDS in two column halves and every output row is summed over
//    its 256 columns in the same fixed order, so identical input rows give
//    bit-identical scores wherever they sit.
#include "rma_device.h"

namespace rma {

constexpr int kRowsWG = 128;
constexpr int kKt = 32;             // contraction depth of one staged slice
constexpr int kStr = kKt + 4;       // LDS row stride (floats) of the m-major / n-major slices
constexpr int kAFloats = kRowsWG * kStr;
constexpr int kBFloats = kMid * kStr;
constexpr int kStageFloats = kAFloats + kBFloats;
constexpr int kZStr = 129;          // stage-1 block: [row][col], floats (one column half)
constexpr int kScoreThreads = 256;

struct ScoreParams {
  const uint16_t *hidden;
  int64_t n_rows, ld_hidden;
  const float *w1, *w2;
  float *scores;
  int64_t ld_scores;
};

// v_mfma_f32_32x32x2f32: lane l supplies A[m = l%32][k = l/32] and B[k = l/32][n = l%32].
// Within a slice of 32 contraction indices, lane half h = l/32 takes indices
// 16h .. 16h+15 over the slice's 16 MFMA steps, so each lane's 16 operands are
// contiguous in the m-major (A) and n-major (B) LDS layouts and load as four
// 16-byte reads.  The same k order is used for A and B, so the products pair up.
__global__ __launch_bounds__(kScoreThreads, 1) void score_kernel(ScoreParams a) {
  __shared__ __align__(16) float smem[2 * kStageFloats];
  __shared__ float w2s[kMid * kGroups];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;  // wave's 64-row half and 128-column half
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRowsWG;

  for (int i = tid; i < kMid * kGroups; i += kScoreThreads) w2s[i] = a.w2[i];

  // staging roles: A (hidden) row am, k half ah (16 values, m-major); B (W1)
  // column bn, all 32 k of the slice (n-major)
  const int am = tid >> 1, ah = tid & 1;
  const bool arow_ok = row0 + am < a.n_rows;
  const uint16_t *arow = a.hidden + (arow_ok ? (row0 + am) : 0) * a.ld_hidden + 16 * ah;
  const int bn = tid;  // one W1 column per thread, all 32 k of the slice

  uint4 ha[2];
  float wb[kKt];
  auto load_stage = [&](int kt) {
    if (arow_ok) {
      ha[0] = *reinterpret_cast<const uint4 *>(arow + kt * kKt);
      ha[1] = *reinterpret_cast<const uint4 *>(arow + kt * kKt + 8);
    } else {
      ha[0] = make_uint4(0, 0, 0, 0);
      ha[1] = ha[0];
    }
    const float *wcol = a.w1 + static_cast<size_t>(kt * kKt) * kMid + bn;
#pragma unroll
    for (int k = 0; k < kKt; ++k) wb[k] = wcol[static_cast<size_t>(k) * kMid];
  };
  auto store_stage = [&](int buf) {
    float *As = smem + buf * kStageFloats;
    float *Bs = As + kAFloats;
    const uint32_t w[8] = {ha[0].x, ha[0].y, ha[0].z, ha[0].w, ha[1].x, ha[1].y, ha[1].z, ha[1].w};
    float4 *ad = reinterpret_cast<float4 *>(As + am * kStr + 16 * ah);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      ad[j] = make_float4(bf16_lo(w[2 * j]), bf16_hi(w[2 * j]), bf16_lo(w[2 * j + 1]),
                          bf16_hi(w[2 * j + 1]));
    float4 *bd = reinterpret_cast<float4 *>(Bs + bn * kStr);
#pragma unroll
    for (int j = 0; j < kKt / 4; ++j)
      bd[j] = make_float4(wb[4 * j], wb[4 * j + 1], wb[4 * j + 2], wb[4 * j + 3]);
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
  const int kh = lane >> 5, ml = lane & 31;
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) load_stage(kt + 1);
    const float *As = smem + (kt & 1) * kStageFloats;
    const float *Bs = As + kAFloats;
    float4 av[2][4], bv[4][4];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        av[r][j] = *reinterpret_cast<const float4 *>(As + (wr * 64 + 32 * r + ml) * kStr + 16 * kh + 4 * j);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bv[c][j] = *reinterpret_cast<const float4 *>(Bs + (wc * 128 + 32 * c + ml) * kStr + 16 * kh + 4 * j);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int j = kk >> 2, e = kk & 3;
      const float a0 = av[0][j][e], a1 = av[1][j][e];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float b = bv[c][j][e];
        acc[0][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b, acc[0][c], 0, 0, 0);
        acc[1][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b, acc[1][c], 0, 0, 0);
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
            const int row = wr * 64 + r * 32 + 8 * (q >> 2) + 4 * kh + (q & 3);
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
