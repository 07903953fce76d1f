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
// One workgroup (256 threads) per (sequence, KV group), so that a CU holds several
// and one's selection overlaps another's copies:
//   1. build the 1280 candidate keys, five per thread, in registers;
//   2. the admission threshold is the min(1024, n_bank + n_pend)-th largest key
//      (equal keys counted): a first pass sorts the candidates into buckets by
//      score, linearly between the segment's smallest and largest score (a
//      monotone map), and finds the bucket holding that rank; its few keys are
//      then ranked against each other directly, or, for a bucket too full (all
//      scores equal, heavy ties), radix selection continues among them byte by
//      byte from the top;
//   3. a bank record survives in place; free slots (evicted slots, then slots
//      >= n_bank) are listed in ascending order by a prefix sum; admitted
//      pending rows, in ascending row order, take the free slots in order;
//   4. only admitted rows move: each wave moves whole rows -- K and V (512 bytes
//      each in BF16, 256 bytes of E4M3 codes in the FP8 variant) one 16-byte piece
//      per lane, 8 rows in flight per lane, with non-temporal loads and stores
//      (the rows are read once and not read again by this launch) -- plus their
//      score, source and, in the FP8 variant, the two row scales;
//   5. a second launch sets n_bank = min(1024, n_bank + n_pend), n_pend = 0, once
//      every group's workgroup has read them.
#include "rma_device.h"

namespace rma {

constexpr int kCand = kBank + kBlock;  // 1280
constexpr int kCommitThreads = 256;
constexpr int kCopyBatch = 8;  // rows in flight per lane of the copy loop

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

// Exclusive prefix sum over the workgroup's 256 threads; every thread must call it
// (it contains workgroup barriers).
__device__ __forceinline__ int exclusive_scan(int v, int *wave_tot, int wave, int lane,
                                              int &total) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int c = wave_tot[w];
    base += w < wave ? c : 0;
    total += c;
  }
  __syncthreads();
  return base + x - v;
}

// Up to RMA_MAX_JOBS layers committed by one launch (blockIdx.y picks the layer).
struct CommitJobs {
  CommitParams job[RMA_MAX_JOBS];
};

template <bool kFp8>
__device__ __forceinline__ void commit_group(const CommitParams &a) {
  constexpr int kRowBytes = kFp8 ? kDim : 2 * kDim;
  constexpr int kPieces = kRowBytes / 16;  // 16-byte pieces per row
  __shared__ uint32_t hist[256];
  __shared__ uint64_t sel_key;
  __shared__ int sel_digit, sel_rank, sel_count;
  __shared__ uint8_t keep[kCand];
  __shared__ int16_t free_list[kBank];
  __shared__ int16_t kidx[kBank];
  __shared__ int16_t adm_slot[kBlock];
  __shared__ int16_t adm_rows[kBlock];
  __shared__ int wave_tot[4];
  __shared__ float red_lo[4], red_hi[4];
  __shared__ uint64_t gather[kCommitThreads];
  __shared__ int gather_n;

  const int b = blockIdx.x / kGroups;
  const int g = blockIdx.x % kGroups;
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int nb = min(max(a.n_bank[b], 0), kBank);
  const int np = min(max(a.n_pend[b], 0), kBlock);
  const int kk = min(kBank, nb + np);
  const size_t sg = static_cast<size_t>(b) * kGroups + g;

  // 1. keys: thread t holds candidates t + 256 r (r < 5; 1280 = 5 x 256)
  constexpr int kPer = kCand / kCommitThreads;
  uint64_t mine[kPer];
  float msc[kPer];
  bool act[kPer];  // a valid candidate still in the running for the threshold
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = t + kCommitThreads * r;
    uint64_t k = 0;
    float sc = 0.f;
    bool v = false;
    if (i < kBank) {
      if (i < nb) {
        sc = a.bank_score[sg * kBank + i];
        k = cand_key(sc, a.bank_src[sg * kBank + i]);
        v = true;
      }
    } else {
      const int tt = i - kBank;
      if (tt < np) {
        sc = a.pend_score[(static_cast<size_t>(b) * kBlock + tt) * kGroups + g];
        k = cand_key(sc, a.pend_src[static_cast<size_t>(b) * kBlock + tt]);
        v = true;
      }
    }
    mine[r] = k;
    msc[r] = sc;
    act[r] = v;
  }

  // 2. threshold: the kk-th largest key (counting equal keys).
  //  a. A first pass sorts the valid candidates into 255 buckets by score, linearly
  //     between the segment's smallest and largest number (NaN scores form a bucket
  //     of their own below them).  The map is monotone, so every key of a higher
  //     bucket is larger than every key of a lower one; the pass picks the bucket
  //     holding rank kk and the rank left inside it.
  //  b. If that bucket holds at most 256 keys, they are gathered and each is ranked
  //     against the others directly.  Otherwise (scores all equal, heavy ties) radix
  //     selection continues among the bucket's keys, byte by byte from the top: each
  //     pass counts, per byte value, the keys that match the bytes chosen so far,
  //     picks the byte under which the target rank falls and carries the rank left
  //     inside it; once that byte holds a single key, that key is the threshold.
  uint64_t thr = 0;
  if (kk > 0) {
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int r = 0; r < kPer; ++r)
      if (act[r] && !__builtin_isnan(msc[r])) {
        lo = fminf(lo, msc[r]);
        hi = fmaxf(hi, msc[r]);
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, off, 64));
      hi = fmaxf(hi, __shfl_xor(hi, off, 64));
    }
    if (lane == 0) {
      red_lo[wave] = lo;
      red_hi[wave] = hi;
    }
    hist[t] = 0;
    if (t == 0) gather_n = 0;
    __syncthreads();
    lo = fminf(fminf(red_lo[0], red_lo[1]), fminf(red_lo[2], red_lo[3]));
    hi = fmaxf(fmaxf(red_hi[0], red_hi[1]), fmaxf(red_hi[2], red_hi[3]));
    const float scale = 254.0f / (hi - lo);
    const bool spread = hi > lo && scale < INFINITY;
    int rank = kk;
    int count = 0x7fffffff;
    if (spread) {
      int bin[kPer];
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const float x = (msc[r] - lo) * scale;  // in [0, 254] (NaN for a NaN score)
        bin[r] = __builtin_isnan(msc[r]) ? 0 : 1 + min(253, static_cast<int>(x));
        if (act[r]) atomicAdd(&hist[bin[r]], 1u);
      }
      __syncthreads();
      // thread t takes bucket 255 - t: the exclusive sum counts the larger ones
      const int c = static_cast<int>(hist[255 - t]);
      int total;
      const int above = exclusive_scan(c, wave_tot, wave, lane, total);
      if (above < rank && above + c >= rank) {
        sel_digit = 255 - t;
        sel_rank = rank - above;
        sel_count = c;
      }
      __syncthreads();
      rank = sel_rank;
      count = sel_count;
#pragma unroll
      for (int r = 0; r < kPer; ++r) act[r] = act[r] && bin[r] == sel_digit;
    }
    if (count <= kCommitThreads) {
      // b. rank the bucket's keys against each other
#pragma unroll
      for (int r = 0; r < kPer; ++r)
        if (act[r]) gather[atomicAdd(&gather_n, 1)] = mine[r];
      __syncthreads();
      if (t < count) {
        const uint64_t k = gather[t];
        int gt = 0, ge = 0;
        for (int j = 0; j < count; ++j) {
          const uint64_t o = gather[j];
          gt += o > k;
          ge += o >= k;
        }
        if (gt < rank && rank <= ge) sel_key = k;
      }
      __syncthreads();
      thr = sel_key;
    } else {
      uint64_t prefix = 0, pmask = 0;
      for (int shift = 56; shift >= 0; shift -= 8) {
        hist[t] = 0;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kPer; ++r)
          if (act[r] && (mine[r] & pmask) == prefix)
            atomicAdd(&hist[static_cast<int>(mine[r] >> shift) & 255], 1u);
        __syncthreads();
        const int c = static_cast<int>(hist[255 - t]);
        int total;
        const int above = exclusive_scan(c, wave_tot, wave, lane, total);
        if (above < rank && above + c >= rank) {
          sel_digit = 255 - t;
          sel_rank = rank - above;
          sel_count = c;
        }
        __syncthreads();
        prefix |= static_cast<uint64_t>(sel_digit) << shift;
        pmask |= static_cast<uint64_t>(255) << shift;
        rank = sel_rank;
        if (sel_count == 1 || shift == 0) {
          if (sel_count == 1) {
#pragma unroll
            for (int r = 0; r < kPer; ++r)
              if (act[r] && (mine[r] & pmask) == prefix) sel_key = mine[r];
            __syncthreads();
            thr = sel_key;
          } else {
            thr = prefix;
          }
          break;
        }
      }
    }
  }

  // 3a. keep flags
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = t + kCommitThreads * r;
    const bool valid = i < kBank ? (i < nb) : (i - kBank < np);
    keep[i] = (kk > 0 && valid && mine[r] >= thr) ? 1 : 0;
  }
  __syncthreads();

  // 3b. free slots, ascending (thread t owns slots 4t..4t+3)
  int fl[4], cnt = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int s = 4 * t + e;
    const bool survive = s < nb && keep[s];
    fl[e] = survive ? 0 : 1;
    cnt += fl[e];
    kidx[s] = survive ? static_cast<int16_t>(s) : static_cast<int16_t>(-1);
  }
  int n_free;
  int r0 = exclusive_scan(cnt, wave_tot, wave, lane, n_free);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (fl[e]) free_list[r0++] = static_cast<int16_t>(4 * t + e);

  // 3c. admitted pending rows, ascending (thread t owns row t)
  const int adm = (t < np && keep[kBank + t]) ? 1 : 0;
  int n_adm;
  const int arank = exclusive_scan(adm, wave_tot, wave, lane, n_adm);
  n_adm = min(n_adm, n_free);
  // (the scan's barriers order the free_list writes above before these reads)
  int16_t slot = -1;
  if (adm && arank < n_free) {
    slot = free_list[arank];
    adm_rows[arank] = static_cast<int16_t>(t);
  }
  adm_slot[t] = slot;
  __syncthreads();
  if (slot >= 0) kidx[slot] = static_cast<int16_t>(kBank + t);
  __syncthreads();

  // 4. outputs and copies
  if (a.keep_idx) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a.keep_idx[sg * kBank + 4 * t + e] = kidx[4 * t + e];
  }
  // Whole rows per wave: an admitted row's K and V are 2 * kPieces 16-byte pieces,
  // one per lane (lanes [0, kPieces): K, [kPieces, 2 kPieces): V), so a wave moves
  // 64 / (2 kPieces) rows per instruction.  Wave w takes rows w, w + 4, ... of the
  // admitted list; each lane keeps kCopyBatch loads in flight before its stores.
  {
    constexpr int kLanesPerRow = 2 * kPieces;             // 64 (BF16) or 32 (FP8)
    constexpr int kRowsPerInst = 64 / kLanesPerRow;       // 1 or 2
    constexpr int kRowsPerPass = 4 * kRowsPerInst;        // rows the 4 waves move per instruction
    const int sub = lane / kLanesPerRow;
    const int piece = lane % kLanesPerRow;
    const bool is_v = piece >= kPieces;
    const size_t off = static_cast<size_t>(piece % kPieces) * 16;
    const uint8_t *src_base = (is_v ? a.pend_v : a.pend_k) + sg * kBlock * kRowBytes + off;
    uint8_t *dst_base = (is_v ? a.bank_v : a.bank_k) + sg * kBank * kRowBytes + off;
    const int first = wave * kRowsPerInst + sub;
    for (int i0 = first; i0 < n_adm; i0 += kRowsPerPass * kCopyBatch) {
      u32x4 buf[kCopyBatch];
#pragma unroll
      for (int u = 0; u < kCopyBatch; ++u) {
        const int i = i0 + u * kRowsPerPass;
        if (i < n_adm) {
          const uint8_t *src = src_base + static_cast<size_t>(adm_rows[i]) * kRowBytes;
          buf[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
        }
      }
#pragma unroll
      for (int u = 0; u < kCopyBatch; ++u) {
        const int i = i0 + u * kRowsPerPass;
        if (i < n_adm) {
          uint8_t *dst = dst_base + static_cast<size_t>(adm_slot[adm_rows[i]]) * kRowBytes;
          __builtin_nontemporal_store(buf[u], reinterpret_cast<u32x4 *>(dst));
        }
      }
    }
  }
  if (t < n_adm) {
    const int row = adm_rows[t];
    const int s = adm_slot[row];
    a.bank_score[sg * kBank + s] = a.pend_score[(static_cast<size_t>(b) * kBlock + row) * kGroups + g];
    a.bank_src[sg * kBank + s] = a.pend_src[static_cast<size_t>(b) * kBlock + row];
    if constexpr (kFp8) {
      a.bank_ks[sg * kBank + s] = a.pend_ks[sg * kBlock + row];
      a.bank_vs[sg * kBank + s] = a.pend_vs[sg * kBlock + row];
    }
  }
}

// One call: the parameters stay in the kernel's own argument registers.
template <bool kFp8>
__global__ __launch_bounds__(kCommitThreads) void commit_kernel(CommitParams a) {
  commit_group<kFp8>(a);
}

// Several layers in one launch (blockIdx.y picks the layer).
template <bool kFp8>
__global__ __launch_bounds__(kCommitThreads) void commit_multi_kernel(CommitJobs jobs) {
  commit_group<kFp8>(jobs.job[blockIdx.y]);
}

// 5. counters, after every group's workgroup has read them (a launch of its own).
struct CounterJobs {
  int32_t *n_bank[RMA_MAX_JOBS];
  int32_t *n_pend[RMA_MAX_JOBS];
};

__global__ __launch_bounds__(256) void commit_counters_kernel(CounterJobs jobs, int batch) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= batch) return;
  int32_t *n_bank = jobs.n_bank[blockIdx.y];
  int32_t *n_pend = jobs.n_pend[blockIdx.y];
  const int nb = min(max(n_bank[b], 0), kBank);
  const int np = min(max(n_pend[b], 0), kBlock);
  n_bank[b] = min(kBank, nb + np);
  n_pend[b] = 0;
}

}  // namespace rma

using namespace rma;

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <bool kFp8>
static rma_status check_commit(const CommitParams &p) {
  if (!p.bank_k || !p.bank_v || !p.bank_score || !p.bank_src || !p.pend_k || !p.pend_v ||
      !p.pend_score || !p.pend_src || !p.n_bank || !p.n_pend)
    return RMA_E_ARG;
  if (kFp8 && (!p.bank_ks || !p.bank_vs || !p.pend_ks || !p.pend_vs)) return RMA_E_ARG;
  const void *al[] = {p.bank_k, p.bank_v, p.pend_k, p.pend_v};
  for (const void *ptr : al)
    if (!aligned16(ptr)) return RMA_E_ALIGN;
  return RMA_OK;
}

template <bool kFp8>
static rma_status launch_commit(const CommitJobs &jobs, int n_jobs, int32_t batch, void *stream) {
  if (batch <= 0 || batch > RMA_MAX_BATCH) return RMA_E_ARG;
  CounterJobs cj{};
  for (int j = 0; j < n_jobs; ++j) {
    const rma_status rc = check_commit<kFp8>(jobs.job[j]);
    if (rc != RMA_OK) return rc;
    cj.n_bank[j] = jobs.job[j].n_bank;
    cj.n_pend[j] = jobs.job[j].n_pend;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned nj = static_cast<unsigned>(n_jobs);
  if (n_jobs == 1)
    hipLaunchKernelGGL(commit_kernel<kFp8>, dim3(batch * kGroups), dim3(kCommitThreads), 0, s,
                       jobs.job[0]);
  else
    hipLaunchKernelGGL(commit_multi_kernel<kFp8>, dim3(batch * kGroups, nj), dim3(kCommitThreads),
                       0, s, jobs);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  hipLaunchKernelGGL(commit_counters_kernel, dim3((batch + 255) / 256, nj), dim3(256), 0, s, cj,
                     batch);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  return RMA_OK;
}

static CommitParams commit_params(const rma_layer_state *st, int32_t *keep_idx) {
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
  return p;
}

extern "C" rma_status rma_commit_topk(const rma_layer_state *st, int32_t batch, int32_t *keep_idx,
                                      void *stream) {
  if (!st) return RMA_E_ARG;
  CommitJobs jobs{};
  jobs.job[0] = commit_params(st, keep_idx);
  return launch_commit<false>(jobs, 1, batch, stream);
}

extern "C" rma_status rma_commit_topk_multi(const rma_layer_state *states, int32_t n_states,
                                            int32_t batch, int32_t *const *keep_idx,
                                            void *stream) {
  if (!states || n_states < 1 || n_states > RMA_MAX_JOBS) return RMA_E_ARG;
  CommitJobs jobs{};
  for (int j = 0; j < n_states; ++j)
    jobs.job[j] = commit_params(&states[j], keep_idx ? keep_idx[j] : nullptr);
  return launch_commit<false>(jobs, n_states, batch, stream);
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
  CommitJobs jobs{};
  jobs.job[0] = p;
  return launch_commit<true>(jobs, 1, batch, stream);
}
