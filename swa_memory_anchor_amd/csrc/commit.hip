// Commit the pending block: per KV group, keep the best 1024 of bank + pending.
//
// neodrop.ai repost of the QbitAI article "内存还会跌吗？KV Cache砍掉99%…", section
// "三段记忆，只记值得记的": every 256 candidates are ranked together with the
// anchors already kept and only the best 1024 survive, each KV group on its own;
// kept anchors are independent and never change.  fluxbbs.com "EdgeRock-4B 开源…",
// section "架构：递归、局部窗口与记忆锚点三件套": groups choose independently and may
// keep the same source positions.
//
// Order: higher score first; equal scores keep the lower source position; -0.0
// equals +0.0; NaN below every number.  Each candidate becomes one 64-bit key
// (order-preserving image of the score in the high word, the complement of the
// source position in the low word), so "better" is "larger key" and the order is
// total whenever sources are distinct within a group.
//
// One workgroup (1024 threads) per sequence; 256 threads per KV group:
//   1. build 1280 keys (2048 with zero padding, below every real key) in LDS;
//   2. bitonic sort, descending; the 1024th key is the admission threshold;
//   3. a bank record survives in place; free slots (evicted slots, then slots
//      >= n_bank) are listed in ascending order by a prefix sum; admitted
//      pending rows, in ascending row order, take the free slots in order;
//   4. only admitted rows move: 512-byte K and V rows are copied in 16-byte
//      pieces (a wave covers one row per pass, 8 passes in flight), plus their
//      score and source;
//   5. n_bank = min(1024, n_bank + n_pend), n_pend = 0.
#include "rma_device.h"

namespace rma {

constexpr int kCand = kBank + kBlock;  // 1280
constexpr int kSortN = 2048;
constexpr int kGroupThreads = 256;
constexpr int kCommitThreads = kGroupThreads * kGroups;
constexpr int kCopyBatch = 8;  // 16-byte copies in flight per thread

struct CommitParams {
  uint16_t *bank_k, *bank_v;
  float *bank_score;
  int32_t *bank_src;
  const uint16_t *pend_k, *pend_v;
  const float *pend_score;
  const int32_t *pend_src;
  int32_t *n_bank, *n_pend;
  int32_t *keep_idx;
};

// Monotone map of IEEE binary32 onto uint32: a < b (as numbers) iff map(a) < map(b);
// both zeros map to the same value; NaN maps to 0, below every number.
__device__ __forceinline__ uint32_t score_order(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t cand_key(float score, int32_t src) {
  return (static_cast<uint64_t>(score_order(score)) << 32) | static_cast<uint32_t>(~src);
}

// Exclusive prefix sum over the 256 threads of one group; every thread of the
// workgroup must call it (it contains workgroup barriers).
__device__ __forceinline__ int group_exclusive_scan(int v, int (*wave_tot)[4], int g, int gw,
                                                    int lane, int &total) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[g][gw] = x;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int c = wave_tot[g][w];
    base += w < gw ? c : 0;
    total += c;
  }
  __syncthreads();
  return base + x - v;
}

__global__ __launch_bounds__(kCommitThreads) void commit_kernel(CommitParams a) {
  __shared__ uint64_t keys[kGroups][kSortN];
  __shared__ uint8_t keep[kGroups][kCand];
  __shared__ int16_t free_list[kGroups][kBank];
  __shared__ int16_t kidx[kGroups][kBank];
  __shared__ int16_t adm_slot[kGroups][kBlock];
  __shared__ int16_t adm_rows[kGroups][kBlock];
  __shared__ int wave_tot[kGroups][4];

  const int b = blockIdx.x;
  const int g = threadIdx.x / kGroupThreads;
  const int t = threadIdx.x % kGroupThreads;
  const int gw = t >> 6;
  const int lane = threadIdx.x & 63;
  const int nb = min(max(a.n_bank[b], 0), kBank);
  const int np = min(max(a.n_pend[b], 0), kBlock);
  const int kk = min(kBank, nb + np);
  const size_t sg = static_cast<size_t>(b) * kGroups + g;

  // 1. keys
  uint64_t mine[5];
#pragma unroll
  for (int r = 0; r < kSortN / kGroupThreads; ++r) {
    const int i = t + kGroupThreads * r;
    uint64_t k = 0;
    if (i < kBank) {
      if (i < nb) k = cand_key(a.bank_score[sg * kBank + i], a.bank_src[sg * kBank + i]);
    } else if (i < kCand) {
      const int tt = i - kBank;
      if (tt < np)
        k = cand_key(a.pend_score[(static_cast<size_t>(b) * kBlock + tt) * kGroups + g],
                     a.pend_src[static_cast<size_t>(b) * kBlock + tt]);
    }
    keys[g][i] = k;
    if (r < 5) mine[r] = k;
  }

  // 2. bitonic sort, descending
  for (int k2 = 2; k2 <= kSortN; k2 <<= 1) {
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kSortN / 2 / kGroupThreads; ++q) {
        const int idx = t + kGroupThreads * q;
        const int i = 2 * j * (idx / j) + (idx % j);
        const int ixj = i + j;
        const uint64_t x = keys[g][i], y = keys[g][ixj];
        const bool desc = (i & k2) == 0;
        if (desc ? (x < y) : (x > y)) {
          keys[g][i] = y;
          keys[g][ixj] = x;
        }
      }
    }
  }
  __syncthreads();
  const uint64_t thr = kk > 0 ? keys[g][kk - 1] : 0;

  // 3a. keep flags
#pragma unroll
  for (int r = 0; r < 5; ++r) {
    const int i = t + kGroupThreads * r;
    const bool valid = i < kBank ? (i < nb) : (i - kBank < np);
    keep[g][i] = (kk > 0 && valid && mine[r] >= thr) ? 1 : 0;
  }
  __syncthreads();

  // 3b. free slots, ascending (thread t owns slots 4t..4t+3)
  int fl[4], cnt = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int s = 4 * t + e;
    const bool survive = s < nb && keep[g][s];
    fl[e] = survive ? 0 : 1;
    cnt += fl[e];
    kidx[g][s] = survive ? static_cast<int16_t>(s) : static_cast<int16_t>(-1);
  }
  int n_free;
  int r0 = group_exclusive_scan(cnt, wave_tot, g, gw, lane, n_free);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (fl[e]) free_list[g][r0++] = static_cast<int16_t>(4 * t + e);

  // 3c. admitted pending rows, ascending (thread t owns row t)
  const int adm = (t < np && keep[g][kBank + t]) ? 1 : 0;
  int n_adm;
  const int arank = group_exclusive_scan(adm, wave_tot, g, gw, lane, n_adm);
  n_adm = min(n_adm, n_free);
  // (the scan's barriers order the free_list writes above before these reads)
  int16_t slot = -1;
  if (adm && arank < n_free) {
    slot = free_list[g][arank];
    adm_rows[g][arank] = static_cast<int16_t>(t);
  }
  adm_slot[g][t] = slot;
  __syncthreads();
  if (slot >= 0) kidx[g][slot] = static_cast<int16_t>(kBank + t);
  __syncthreads();

  // 4. outputs and copies
  if (a.keep_idx) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a.keep_idx[sg * kBank + 4 * t + e] = kidx[g][4 * t + e];
  }
  // 16-byte pieces: 64 per admitted row (32 of K, 32 of V).  Each thread issues
  // kCopyBatch loads before its stores, so a group waits for at most
  // 64 * 256 / (256 * kCopyBatch) round trips to memory instead of one per piece.
  const int pieces = n_adm * 64;
  for (int w0 = 0; w0 < pieces; w0 += kGroupThreads * kCopyBatch) {
    u32x4 buf[kCopyBatch];
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) {
      // past the end, repeat the last piece: the same bytes go to the same place
      const int w = min(w0 + t + u * kGroupThreads, pieces - 1);
      const int row = adm_rows[g][w >> 6];
      const int part = w & 63;
      const uint16_t *src = (part >= 32 ? a.pend_v : a.pend_k) + (sg * kBlock + row) * kDim +
                            (part & 31) * 8;
      buf[u] = *reinterpret_cast<const u32x4 *>(src);
    }
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) {
      const int w = min(w0 + t + u * kGroupThreads, pieces - 1);
      const int row = adm_rows[g][w >> 6];
      const int part = w & 63;
      const int sl = adm_slot[g][row];
      uint16_t *dst = (part >= 32 ? a.bank_v : a.bank_k) + (sg * kBank + sl) * kDim +
                      (part & 31) * 8;
      *reinterpret_cast<u32x4 *>(dst) = buf[u];
    }
  }
  if (t < n_adm) {
    const int row = adm_rows[g][t];
    const int s = adm_slot[g][row];
    a.bank_score[sg * kBank + s] = a.pend_score[(static_cast<size_t>(b) * kBlock + row) * kGroups + g];
    a.bank_src[sg * kBank + s] = a.pend_src[static_cast<size_t>(b) * kBlock + row];
  }

  // 5. counters, after every group has read them
  __syncthreads();
  if (threadIdx.x == 0) {
    a.n_bank[b] = kk;
    a.n_pend[b] = 0;
  }
}

}  // namespace rma

using namespace rma;

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

extern "C" rma_status rma_commit_topk(const rma_layer_state *st, int32_t batch, int32_t *keep_idx,
                                      void *stream) {
  if (!st || batch <= 0 || batch > RMA_MAX_BATCH) return RMA_E_ARG;
  if (!st->bank_k || !st->bank_v || !st->bank_score || !st->bank_src || !st->pend_k ||
      !st->pend_v || !st->pend_score || !st->pend_src || !st->n_bank || !st->n_pend)
    return RMA_E_ARG;
  const void *al[] = {st->bank_k, st->bank_v, st->pend_k, st->pend_v};
  for (const void *p : al)
    if (!aligned16(p)) return RMA_E_ALIGN;
  CommitParams p;
  p.bank_k = st->bank_k;
  p.bank_v = st->bank_v;
  p.bank_score = st->bank_score;
  p.bank_src = st->bank_src;
  p.pend_k = st->pend_k;
  p.pend_v = st->pend_v;
  p.pend_score = st->pend_score;
  p.pend_src = st->pend_src;
  p.n_bank = st->n_bank;
  p.n_pend = st->n_pend;
  p.keep_idx = keep_idx;
  hipLaunchKernelGGL(commit_kernel, dim3(batch), dim3(kCommitThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  return RMA_OK;
}
