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
//    a 64 x 128 block = 2 x 4 accumulators of 32 x 32 (32-row tiles for calls too
//    small to give every CU a 128-row tile);
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

constexpr int kKt = 32;             // contraction depth of one staged slice
constexpr int kStr = kKt + 4;       // LDS row stride (floats) of the m-major / n-major slices
constexpr int kZStr = 129;          // stage-1 block: [row][col], floats (one column half)
constexpr int kScoreThreads = 256;
constexpr int kMaxRowsWG = 128;
constexpr int kStageFloats = kMaxRowsWG * kStr + kMid * kStr;

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
//
// Tile shapes: the 4 waves are arranged WR x (4/WR); each wave owns RB row blocks
// and CB column blocks of 32 x 32.  Large calls use 128-row tiles (WR=2, RB=2,
// CB=4); calls with fewer such tiles than CUs use 64-row tiles (WR=2, RB=1, CB=4)
// or, fewer still, 32-row tiles (WR=1, RB=1, CB=2).  All run the same instruction
// sequence per output element, so results do not depend on the tile shape.
// Up to RMA_MAX_JOBS independent calls of the same row count in one launch
// (blockIdx.y picks the call): the layers of a block, scored together.
struct ScoreJobs {
  ScoreParams job[RMA_MAX_JOBS];
};

template <int WR, int RB, int CB>
__global__ __launch_bounds__(kScoreThreads, 1) void score_kernel(ScoreJobs jobs) {
  const ScoreParams &a = jobs.job[blockIdx.y];
  constexpr int WC = 4 / WR;
  constexpr int kRows = 32 * RB * WR;
  constexpr int kColsW = 32 * CB;  // columns per wave
  static_assert(kColsW * WC == kMid, "waves cover the 256 columns");
  constexpr int kAFloats = kRows * kStr;
  constexpr int kSF = kAFloats + kMid * kStr;
  constexpr int kTpr = kScoreThreads / kRows;  // staging threads per hidden row
  constexpr int kKpt = kKt / kTpr;             // k values each of them stages (16, 8 or 4)
  __shared__ __align__(16) float smem[2 * kStageFloats];
  __shared__ float w2s[kMid * kGroups];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave / WC, wc = wave % WC;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRows;

  for (int i = tid; i < kMid * kGroups; i += kScoreThreads) w2s[i] = a.w2[i];

  // staging roles: A (hidden) row am, k chunk ah (kKpt values, m-major); B (W1)
  // column bn, all 32 k of the slice (n-major)
  const int am = tid / kTpr, ah = tid % kTpr;
  const bool arow_ok = row0 + am < a.n_rows;
  const uint16_t *arow = a.hidden + (arow_ok ? (row0 + am) : 0) * a.ld_hidden + kKpt * ah;
  const int bn = tid;

  uint32_t ha[kKpt / 2];
  float wb[kKt];
  auto load_stage = [&](int kt) {
    if constexpr (kKpt == 16) {
      uint4 u0 = make_uint4(0, 0, 0, 0), u1 = u0;
      if (arow_ok) {
        u0 = *reinterpret_cast<const uint4 *>(arow + kt * kKt);
        u1 = *reinterpret_cast<const uint4 *>(arow + kt * kKt + 8);
      }
      ha[0] = u0.x; ha[1] = u0.y; ha[2] = u0.z; ha[3] = u0.w;
      ha[4] = u1.x; ha[5] = u1.y; ha[6] = u1.z; ha[7] = u1.w;
    } else if constexpr (kKpt == 8) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (arow_ok) u = *reinterpret_cast<const uint4 *>(arow + kt * kKt);
      ha[0] = u.x; ha[1] = u.y; ha[2] = u.z; ha[3] = u.w;
    } else {
      static_assert(kKpt == 4, "staging chunk");
      uint2 u = make_uint2(0, 0);
      if (arow_ok) u = *reinterpret_cast<const uint2 *>(arow + kt * kKt);
      ha[0] = u.x;
      ha[1] = u.y;
    }
    const float *wcol = a.w1 + static_cast<size_t>(kt * kKt) * kMid + bn;
#pragma unroll
    for (int k = 0; k < kKt; ++k) wb[k] = wcol[static_cast<size_t>(k) * kMid];
  };
  auto store_stage = [&](int buf) {
    float *As = smem + buf * kSF;
    float *Bs = As + kAFloats;
    float4 *ad = reinterpret_cast<float4 *>(As + am * kStr + kKpt * ah);
#pragma unroll
    for (int j = 0; j < kKpt / 4; ++j)
      ad[j] = make_float4(bf16_lo(ha[2 * j]), bf16_hi(ha[2 * j]), bf16_lo(ha[2 * j + 1]),
                          bf16_hi(ha[2 * j + 1]));
    float4 *bd = reinterpret_cast<float4 *>(Bs + bn * kStr);
#pragma unroll
    for (int j = 0; j < kKt / 4; ++j)
      bd[j] = make_float4(wb[4 * j], wb[4 * j + 1], wb[4 * j + 2], wb[4 * j + 3]);
  };

  f32x16 acc[RB][CB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[r][c][q] = 0.f;

  constexpr int nkt = kHidden / kKt;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  const int kh = lane >> 5, ml = lane & 31;
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) load_stage(kt + 1);
    const float *As = smem + (kt & 1) * kSF;
    const float *Bs = As + kAFloats;
    float4 av[RB][4], bv[CB][4];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        av[r][j] = *reinterpret_cast<const float4 *>(
            As + (wr * 32 * RB + 32 * r + ml) * kStr + 16 * kh + 4 * j);
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bv[c][j] = *reinterpret_cast<const float4 *>(
            Bs + (wc * kColsW + 32 * c + ml) * kStr + 16 * kh + 4 * j);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int j = kk >> 2, e = kk & 3;
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const float b = bv[c][j][e];
#pragma unroll
        for (int r = 0; r < RB; ++r)
          acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[r][j][e], b, acc[r][c], 0, 0, 0);
      }
    }
    if (kt + 1 < nkt) store_stage((kt + 1) & 1);
    __syncthreads();
  }

  // Stage 2: s[row][g] = sum_{n=0..255} Z[row][n] * W2[n][g], n ascending, passed
  // through LDS in two column halves.
  float *Z = smem;
  constexpr int kOuts = kRows * kGroups;  // outputs of the tile
  constexpr int kPerThread = (kOuts + kScoreThreads - 1) / kScoreThreads;  // 2 or 1
  const int srow = tid % kRows;
  const int sg = (tid / kRows) * kPerThread;  // first group of this thread
  const bool active = sg < kGroups;
  float sacc[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) sacc[i] = 0.f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wc * kColsW / 128 == half) {
      const int cofs = wc * kColsW - half * 128;
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int row = wr * 32 * RB + r * 32 + 8 * (q >> 2) + 4 * kh + (q & 3);
            Z[row * kZStr + cofs + 32 * c + ml] = acc[r][c][q];
          }
    }
    __syncthreads();
    if (active) {
      const float *zr = Z + srow * kZStr;
      const float *w2h = w2s + half * 128 * kGroups;
      for (int n = 0; n < 128; ++n) {
        const float z = zr[n];
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) sacc[i] = fmaf(z, w2h[n * kGroups + sg + i], sacc[i]);
      }
    }
    __syncthreads();
  }
  if (active && row0 + srow < a.n_rows) {
    float *out = a.scores + (row0 + srow) * a.ld_scores + sg;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) out[i] = sacc[i];
  }
}

}  // namespace rma

using namespace rma;

// Validate one call's arguments (shared by the single and the multi-call entry).
static rma_status check_score(const uint16_t *hidden, int64_t n_rows, int64_t ld_hidden,
                              const float *w1, const float *w2, const float *scores,
                              int64_t ld_scores) {
  if (n_rows < 0 || !w1 || !w2) return RMA_E_ARG;
  if (n_rows == 0) return RMA_OK;
  if (!hidden || !scores) return RMA_E_ARG;
  if (ld_hidden < kHidden || ld_scores < kGroups) return RMA_E_ARG;
  if ((ld_hidden % 8) != 0 || (ld_scores % 4) != 0) return RMA_E_ALIGN;
  if ((reinterpret_cast<uintptr_t>(hidden) & 15u) || (reinterpret_cast<uintptr_t>(w1) & 15u) ||
      (reinterpret_cast<uintptr_t>(scores) & 15u))
    return RMA_E_ALIGN;
  return RMA_OK;
}

static rma_status launch_score(const ScoreJobs &jobs, int n_jobs, int64_t n_rows, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The largest row tile that still gives every CU (256) a workgroup: 128 rows,
  // then 64, then 32 (a larger tile reads W1 fewer times per row).
  const int64_t big = (n_rows + 127) / 128;
  const int64_t mid = (n_rows + 63) / 64;
  const unsigned nj = static_cast<unsigned>(n_jobs);
  if (big >= 256) {
    if (big > 0x7fffffff) return RMA_E_ARG;
    hipLaunchKernelGGL((score_kernel<2, 2, 4>), dim3(static_cast<unsigned>(big), nj),
                       dim3(kScoreThreads), 0, s, jobs);
  } else if (mid >= 256) {
    hipLaunchKernelGGL((score_kernel<2, 1, 4>), dim3(static_cast<unsigned>(mid), nj),
                       dim3(kScoreThreads), 0, s, jobs);
  } else {
    const int64_t small = (n_rows + 31) / 32;
    hipLaunchKernelGGL((score_kernel<1, 1, 2>), dim3(static_cast<unsigned>(small), nj),
                       dim3(kScoreThreads), 0, s, jobs);
  }
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  return RMA_OK;
}

extern "C" rma_status rma_score(const uint16_t *hidden, int64_t n_rows, int64_t ld_hidden,
                                const float *w1, const float *w2, float *scores,
                                int64_t ld_scores, void *stream) {
  const rma_status rc = check_score(hidden, n_rows, ld_hidden, w1, w2, scores, ld_scores);
  if (rc != RMA_OK || n_rows == 0) return rc;
  ScoreJobs jobs{};
  jobs.job[0] = ScoreParams{hidden, n_rows, ld_hidden, w1, w2, scores, ld_scores};
  return launch_score(jobs, 1, n_rows, stream);
}

extern "C" rma_status rma_score_multi(const rma_score_job *jobs, int32_t n_jobs, int64_t n_rows,
                                      int64_t ld_hidden, int64_t ld_scores, void *stream) {
  if (!jobs || n_jobs < 1 || n_jobs > RMA_MAX_JOBS) return RMA_E_ARG;
  ScoreJobs sj{};
  for (int j = 0; j < n_jobs; ++j) {
    const rma_score_job &jb = jobs[j];
    const rma_status rc = check_score(jb.hidden, n_rows, ld_hidden, jb.w1, jb.w2, jb.scores,
                                      ld_scores);
    if (rc != RMA_OK) return rc;
    sj.job[j] = ScoreParams{jb.hidden, n_rows, ld_hidden, jb.w1, jb.w2, jb.scores, ld_scores};
  }
  if (n_rows == 0) return RMA_OK;
  return launch_score(sj, n_jobs, n_rows, stream);
}
