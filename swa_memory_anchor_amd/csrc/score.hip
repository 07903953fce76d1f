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
//  * one workgroup (4 waves) per 256-row tile and all 256 columns; each wave owns
//    a 128 x 128 block = 4 x 4 accumulators of 32 x 32 (256 accumulator registers
//    per lane), so W1 is read once per 256 rows and each staged slice feeds 256
//    MFMAs per wave; calls too small to give every CU a 256-row tile use 128-, 64-
//    or 32-row tiles;
//  * K is walked in slices of 32: BF16 rows are widened (exactly) to FP32 while
//    being staged in LDS row-major (m-major), W1 is staged column-major (n-major);
//    each lane's 16 operands of a slice are then contiguous, so a slice's operands
//    come in with 16-byte LDS reads (32 per slice on 256-row tiles) and its MFMAs
//    issue back to back; two LDS buffers, the next slice's global loads in flight
//    meanwhile;
//  * stage 2 (x W2, 256 -> 4) is fused: the rows x 256 block of stage-1 results is
//    passed through LDS in two column halves and every output row is summed over
//    its 256 columns in the same fixed order, so identical input rows give
//    bit-identical scores wherever they sit.
// Calls too small to give every CU a tile even at 32 rows (a 256-token block of
// a batch-1 stream: 8 tiles per layer) are bound by one CU's MFMA rate per tile.
// With a workspace they take a split path instead: one wave per 32 x 32 block of
// stage-1 results, its operands loaded straight from global memory (four slices
// in flight, no LDS, no barrier), the block written to the workspace; a second
// launch then sums each row over its 256 columns in the same order as above.
// Every stage-1 element is the same MFMA chain in both paths, so the scores are
// bit-identical to those of the one-launch path.
#include "rma_device.h"

namespace rma {

constexpr int kKt = 32;             // contraction depth of one staged slice
constexpr int kStr = kKt + 4;       // LDS row stride (floats) of the m-major / n-major slices
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
//
// Tile shapes: the 4 waves are arranged WR x (4/WR); each wave owns RB row blocks
// and CB column blocks of 32 x 32.  Large calls use 256-row tiles (WR=2, RB=4,
// CB=4); calls with fewer such tiles than CUs use 128-row tiles (WR=2, RB=2, CB=4),
// 64-row tiles (WR=2, RB=1, CB=4) or, fewer still, 32-row tiles (WR=1, RB=1,
// CB=2).  All run the same instruction sequence per output element, so results do
// not depend on the tile shape.
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
  constexpr int kKpt = kKt / kTpr;             // k values each of them stages (32, 16, 8 or 4)
  static_assert(kRows * kZStr <= 2 * kSF, "the stage-1 block fits in the staging buffers");
  __shared__ __align__(16) float smem[2 * kSF];
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
    if constexpr (kKpt == 32) {
      uint4 u[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                    make_uint4(0, 0, 0, 0)};
      if (arow_ok) {
#pragma unroll
        for (int q = 0; q < 4; ++q) u[q] = *reinterpret_cast<const uint4 *>(arow + kt * kKt + 8 * q);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ha[4 * q] = u[q].x; ha[4 * q + 1] = u[q].y; ha[4 * q + 2] = u[q].z; ha[4 * q + 3] = u[q].w;
      }
    } else if constexpr (kKpt == 16) {
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

// Split path, stage 1: workgroup b takes call b % n_jobs (with 8 calls, every
// wave of a call runs on one XCD); its wave w takes task t = (b / n_jobs) *
// waves + w of that call: 32-row tile t / 8, 32-column block t % 8.  Lane l supplies A[m = l%32][k] and B[k][n = l%32]
// for k = 16h .. 16h+15 of each 32-deep slice (h = l/32), exactly the operand
// order of score_kernel, so every element sees the same MFMA sequence.  Rows past
// n_rows load the last row (they are never stored); each slice's loads are
// unconditional, the last ones re-reading the final slice, so the wait for a
// slice covers only that slice.
#ifndef RMA_SCORE_SPLIT_WAVES
#define RMA_SCORE_SPLIT_WAVES 1
#endif
#ifndef RMA_SCORE_SPLIT_DEPTH
#define RMA_SCORE_SPLIT_DEPTH 4
#endif
constexpr int kSplitDepth = RMA_SCORE_SPLIT_DEPTH;  // slices in flight per wave (18 loads each)
constexpr int kColBlocks = kMid / 32;
constexpr int kSplitWaves = RMA_SCORE_SPLIT_WAVES;  // waves (column blocks) per workgroup
static_assert(kColBlocks % kSplitWaves == 0, "a workgroup's waves share one row tile");

__global__ __launch_bounds__(64 * kSplitWaves, 1) void score_split_kernel(ScoreJobs jobs, float *z,
                                                                          int n_jobs) {
  const int job = blockIdx.x % n_jobs;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int task = (blockIdx.x / n_jobs) * kSplitWaves + wave;
  const ScoreParams &a = jobs.job[job];
  const int cb = task % kColBlocks, rt = task / kColBlocks;
  const int lane = threadIdx.x & 63, ml = lane & 31, kh = lane >> 5;
  const int64_t row = min(static_cast<int64_t>(rt) * 32 + ml, a.n_rows - 1);
  const uint16_t *hp = a.hidden + row * a.ld_hidden + 16 * kh;
  const float *wp = a.w1 + static_cast<size_t>(16 * kh) * kMid + 32 * cb + ml;
  constexpr int nkt = kHidden / kKt;
  static_assert(nkt % kSplitDepth == 0, "whole rounds of the slice ring");

  uint4 ra[kSplitDepth][2];
  float rb[kSplitDepth][16];
  // every load fenced: the ring's prologue and its refills then issue the 18 loads
  // of a slice in one order (the order of use), which is what lets the waits at the
  // loop head count only the slice being used
  auto load = [&](int d, int kt) {
    const uint16_t *h = hp + kt * kKt;
    const float *wk = wp + static_cast<size_t>(kt * kKt) * kMid;
    ra[d][0] = *reinterpret_cast<const uint4 *>(h);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      rb[d][kk] = wk[static_cast<size_t>(kk) * kMid];
      __builtin_amdgcn_sched_barrier(0);
    }
    ra[d][1] = *reinterpret_cast<const uint4 *>(h + 8);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 8; kk < 16; ++kk) {
      rb[d][kk] = wk[static_cast<size_t>(kk) * kMid];
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  f32x16 acc;
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.f;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < kSplitDepth; ++d) load(d, d);
  for (int kt0 = 0; kt0 < nkt; kt0 += kSplitDepth) {
#pragma unroll
    for (int d = 0; d < kSplitDepth; ++d) {
      float av[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t u0 = j == 0 ? ra[d][0].x : j == 1 ? ra[d][0].y : j == 2 ? ra[d][0].z : ra[d][0].w;
        const uint32_t u1 = j == 0 ? ra[d][1].x : j == 1 ? ra[d][1].y : j == 2 ? ra[d][1].z : ra[d][1].w;
        av[2 * j] = bf16_lo(u0);
        av[2 * j + 1] = bf16_hi(u0);
        av[8 + 2 * j] = bf16_lo(u1);
        av[8 + 2 * j + 1] = bf16_hi(u1);
      }
      // all 16 operands widened first, then the slice's MFMAs back to back: a VALU
      // or load instruction between two MFMAs of the chain costs more than it hides
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < 16; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[kk], rb[d][kk], acc, 0, 0, 0);
      // the scheduler would otherwise sink each refill next to its use
      __builtin_amdgcn_sched_barrier(0);
      load(d, min(kt0 + d + kSplitDepth, nkt - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // acc[q] is Z[32 rt + 8 (q/4) + 4 h + q%4][32 cb + l%32]
  float *zc = z + static_cast<size_t>(job) * a.n_rows * kMid + 32 * cb + ml;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int64_t r = static_cast<int64_t>(rt) * 32 + 8 * (q >> 2) + 4 * kh + (q & 3);
    if (r < a.n_rows) zc[r * kMid] = acc[q];
  }
}

// Split path, stage 2: one thread per row of call blockIdx.y; s[row][g] =
// sum_{n=0..255} Z[row][n] * W2[n][g], n ascending, the chain of score_kernel.
// The tile's 64 rows come into LDS with coalesced loads (load i of every lane
// reads row i, all 64 in flight: the rows were written by other XCDs), then each
// thread walks its row in a short loop.
constexpr int kZRow = kMid + 4;  // padded LDS row (floats): 16-byte reads down a column hit distinct banks

__global__ __launch_bounds__(64) void score_split_sum_kernel(ScoreJobs jobs, const float *z) {
  const ScoreParams &a = jobs.job[blockIdx.y];
  __shared__ __align__(16) float zs[64 * kZRow];
  __shared__ __align__(16) float w2s[kMid * kGroups];
  const int t = threadIdx.x;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int nr = static_cast<int>(min(static_cast<int64_t>(64), a.n_rows - r0));
  // a buffer resource over the tile's rows: rows past n_rows read as zeros
  const __amdgpu_buffer_rsrc_t zr_all = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(z + (static_cast<size_t>(blockIdx.y) * a.n_rows + r0) * kMid), 0,
      nr * kMid * static_cast<int>(sizeof(float)), 0x00020000);
  using u32x4 = decltype(__builtin_amdgcn_raw_buffer_load_b128(zr_all, 0, 0, 0));
  u32x4 v[64];
#pragma unroll
  for (int i = 0; i < 64; ++i)
    v[i] = __builtin_amdgcn_raw_buffer_load_b128(zr_all, 16 * t, i * kMid * 4, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kMid * kGroups / 64; ++i) w2s[i * 64 + t] = a.w2[i * 64 + t];
#pragma unroll
  for (int i = 0; i < 64; ++i)
    *reinterpret_cast<u32x4 *>(zs + i * kZRow + 4 * t) = v[i];
  __syncthreads();
  if (t >= nr) return;
  const float *zr = zs + t * kZRow;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  static_assert(kGroups == 4, "four scores per row");
#pragma unroll 2
  for (int n4 = 0; n4 < kMid / 4; ++n4) {
    const float4 zz = *reinterpret_cast<const float4 *>(zr + 4 * n4);
    const float e4[4] = {zz.x, zz.y, zz.z, zz.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float4 w = *reinterpret_cast<const float4 *>(w2s + (4 * n4 + e) * kGroups);
      s0 = fmaf(e4[e], w.x, s0);
      s1 = fmaf(e4[e], w.y, s1);
      s2 = fmaf(e4[e], w.z, s2);
      s3 = fmaf(e4[e], w.w, s3);
    }
  }
  *reinterpret_cast<float4 *>(a.scores + (r0 + t) * a.ld_scores) = make_float4(s0, s1, s2, s3);
}

}  // namespace rma

using namespace rma;

// The split path serves calls whose 32-row tiles, over all calls, number at most
// one per CU; it needs n_jobs * n_rows stage-1 rows of workspace.
static bool score_takes_split(int64_t n_jobs, int64_t n_rows) {
  return n_rows > 0 && n_jobs * ((n_rows + 31) / 32) <= 256;
}

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
  // The largest row tile that still gives every CU (256) a workgroup: 256 rows,
  // then 128, 64, 32 (a larger tile reads W1 fewer times per row).
  const int64_t huge = (n_rows + 255) / 256;
  const int64_t big = (n_rows + 127) / 128;
  const int64_t mid = (n_rows + 63) / 64;
  const unsigned nj = static_cast<unsigned>(n_jobs);
  if (huge >= 256) {
    if (huge > 0x7fffffff) return RMA_E_ARG;
    hipLaunchKernelGGL((score_kernel<2, 4, 4>), dim3(static_cast<unsigned>(huge), nj),
                       dim3(kScoreThreads), 0, s, jobs);
  } else if (big >= 256) {
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

static rma_status collect_jobs(const rma_score_job *jobs, int32_t n_jobs, int64_t n_rows,
                               int64_t ld_hidden, int64_t ld_scores, ScoreJobs &sj) {
  if (!jobs || n_jobs < 1 || n_jobs > RMA_MAX_JOBS) return RMA_E_ARG;
  for (int j = 0; j < n_jobs; ++j) {
    const rma_score_job &jb = jobs[j];
    const rma_status rc = check_score(jb.hidden, n_rows, ld_hidden, jb.w1, jb.w2, jb.scores,
                                      ld_scores);
    if (rc != RMA_OK) return rc;
    sj.job[j] = ScoreParams{jb.hidden, n_rows, ld_hidden, jb.w1, jb.w2, jb.scores, ld_scores};
  }
  return RMA_OK;
}

extern "C" rma_status rma_score_multi(const rma_score_job *jobs, int32_t n_jobs, int64_t n_rows,
                                      int64_t ld_hidden, int64_t ld_scores, void *stream) {
  ScoreJobs sj{};
  const rma_status rc = collect_jobs(jobs, n_jobs, n_rows, ld_hidden, ld_scores, sj);
  if (rc != RMA_OK || n_rows == 0) return rc;
  return launch_score(sj, n_jobs, n_rows, stream);
}

extern "C" size_t rma_score_workspace_bytes(int32_t n_jobs, int64_t n_rows) {
  if (n_jobs < 1 || n_jobs > RMA_MAX_JOBS || !score_takes_split(n_jobs, n_rows)) return 0;
  return static_cast<size_t>(n_jobs) * static_cast<size_t>(n_rows) * kMid * sizeof(float);
}

extern "C" rma_status rma_score_multi_ws(const rma_score_job *jobs, int32_t n_jobs, int64_t n_rows,
                                         int64_t ld_hidden, int64_t ld_scores, void *workspace,
                                         size_t workspace_bytes, void *stream) {
  ScoreJobs sj{};
  const rma_status rc = collect_jobs(jobs, n_jobs, n_rows, ld_hidden, ld_scores, sj);
  if (rc != RMA_OK || n_rows == 0) return rc;
  if (!score_takes_split(n_jobs, n_rows)) return launch_score(sj, n_jobs, n_rows, stream);
  if (!workspace || workspace_bytes < rma_score_workspace_bytes(n_jobs, n_rows))
    return RMA_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 15u) return RMA_E_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *z = static_cast<float *>(workspace);
  const unsigned tiles = static_cast<unsigned>((n_rows + 31) / 32);
  hipLaunchKernelGGL(score_split_kernel,
                     dim3(static_cast<unsigned>(n_jobs) * tiles * (kColBlocks / kSplitWaves)),
                     dim3(64 * kSplitWaves), 0, s, sj, z, static_cast<int>(n_jobs));
  hipLaunchKernelGGL(score_split_sum_kernel,
                     dim3(static_cast<unsigned>((n_rows + 63) / 64), static_cast<unsigned>(n_jobs)),
                     dim3(64), 0, s, sj, static_cast<const float *>(z));
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  return RMA_OK;
}
