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
//   4. only admitted rows move: K and V rows (512 bytes in BF16, 256 bytes of
//      E4M3 codes in the FP8 variant) are copied in 16-byte pieces (8 in flight
//      per thread), plus their score, source and, in the FP8 variant, the two
//      row scales;
//   5. n_bank = min(1024, n_bank + n_pend), n_pend = 0.
#include "rma_device.h"

namespace rma {

constexpr int kCand = kBank + kBlock;  // 1280
constexpr int kSortN = 2048;
constexpr int kGroupThreads = 256;
constexpr int kCommitThreads = kGroupThreads * kGroups;
constexpr int kCopyBatch = 8;  // 16-byte copies in flight per thread

// K/V rows are BF16 (512 bytes) or, in the FP8 variant, E4M3 codes (256 bytes)
// with one FP32 scale per row (*_ks, *_vs), which moves with the row.
struct CommitParams {
  uint8_t *bank_k, *bank_v;
  float *bank_ks, *bank_vs;
  float *bank_score;
  int32_t *bank_src;
  const uint8_t *pend_k, *pend_v;
  const float *pend_ks, *pend_vs;
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

template <bool kFp8>
__global__ __launch_bounds__(kCommitThreads) void commit_kernel(CommitParams a) {
  constexpr int kRowBytes = kFp8 ? kDim : 2 * kDim;
  constexpr int kPieces = kRowBytes / 16;  // 16-byte pieces per row
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
  // 16-byte pieces: 2 * kPieces per admitted row (K then V).  Each thread issues
  // kCopyBatch loads before its stores, so a group waits for a handful of round
  // trips to memory instead of one per piece.
  const int pieces = n_adm * 2 * kPieces;
  for (int w0 = 0; w0 < pieces; w0 += kGroupThreads * kCopyBatch) {
    u32x4 buf[kCopyBatch];
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) {
      // past the end, repeat the last piece: the same bytes go to the same place
      const int w = min(w0 + t + u * kGroupThreads, pieces - 1);
      const int row = adm_rows[g][w / (2 * kPieces)];
      const int part = w % (2 * kPieces);
      const uint8_t *src = (part >= kPieces ? a.pend_v : a.pend_k) +
                           (sg * kBlock + row) * kRowBytes + (part % kPieces) * 16;
      buf[u] = *reinterpret_cast<const u32x4 *>(src);
    }
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) {
      const int w = min(w0 + t + u * kGroupThreads, pieces - 1);
      const int row = adm_rows[g][w / (2 * kPieces)];
      const int part = w % (2 * kPieces);
      const int sl = adm_slot[g][row];
      uint8_t *dst = (part >= kPieces ? a.bank_v : a.bank_k) + (sg * kBank + sl) * kRowBytes +
                     (part % kPieces) * 16;
      *reinterpret_cast<u32x4 *>(dst) = buf[u];
    }
  }
  if (t < n_adm) {
    const int row = adm_rows[g][t];
    const int s = adm_slot[g][row];
    a.bank_score[sg * kBank + s] = a.pend_score[(static_cast<size_t>(b) * kBlock + row) * kGroups + g];
    a.bank_src[sg * kBank + s] = a.pend_src[static_cast<size_t>(b) * kBlock + row];
    if constexpr (kFp8) {
      a.bank_ks[sg * kBank + s] = a.pend_ks[sg * kBlock + row];
      a.bank_vs[sg * kBank + s] = a.pend_vs[sg * kBlock + row];
    }
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

template <bool kFp8>
static rma_status launch_commit(const CommitParams &p, int32_t batch, void *stream) {
  if (batch <= 0 || batch > RMA_MAX_BATCH) return RMA_E_ARG;
  if (!p.bank_k || !p.bank_v || !p.bank_score || !p.bank_src || !p.pend_k || !p.pend_v ||
      !p.pend_score || !p.pend_src || !p.n_bank || !p.n_pend)
    return RMA_E_ARG;
  if (kFp8 && (!p.bank_ks || !p.bank_vs || !p.pend_ks || !p.pend_vs)) return RMA_E_ARG;
  const void *al[] = {p.bank_k, p.bank_v, p.pend_k, p.pend_v};
  for (const void *ptr : al)
    if (!aligned16(ptr)) return RMA_E_ALIGN;
  hipLaunchKernelGGL(commit_kernel<kFp8>, dim3(batch), dim3(kCommitThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  return RMA_OK;
}

extern "C" rma_status rma_commit_topk(const rma_layer_state *st, int32_t batch, int32_t *keep_idx,
                                      void *stream) {
  if (!st) return RMA_E_ARG;
  CommitParams p{};
  p.bank_k = reinterpret_cast<uint8_t *>(st->bank_k);
  p.bank_v = reinterpret_cast<uint8_t *>(st->bank_v);
  p.bank_score = st->bank_score;
  p.bank_src = st->bank_src;
  p.pend_k = reinterpret_cast<const uint8_t *>(st->pend_k);
  p.pend_v = reinterpret_cast<const uint8_t *>(st->pend_v);
  p.pend_score = st->pend_score;
  p.pend_src = st->pend_src;
  p.n_bank = st->n_bank;
  p.n_pend = st->n_pend;
  p.keep_idx = keep_idx;
  return launch_commit<false>(p, batch, stream);
}

extern "C" rma_status rma_commit_topk_fp8(const rma_layer_state_fp8 *st, int32_t batch,
                                          int32_t *keep_idx, void *stream) {
  if (!st) return RMA_E_ARG;
  CommitParams p{};
  p.bank_k = st->bank_k;
  p.bank_v = st->bank_v;
  p.bank_ks = st->bank_ks;
  p.bank_vs = st->bank_vs;
  p.bank_score = st->bank_score;
  p.bank_src = st->bank_src;
  p.pend_k = st->pend_k;
  p.pend_v = st->pend_v;
  p.pend_ks = st->pend_ks;
  p.pend_vs = st->pend_vs;
  p.pend_score = st->pend_score;
  p.pend_src = st->pend_src;
  p.n_bank = st->n_bank;
  p.n_pend = st->n_pend;
  p.keep_idx = keep_idx;
  return launch_commit<true>(p, batch, stream);
}
