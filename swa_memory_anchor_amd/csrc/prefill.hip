// Chunked prefill of one SWA||RMA layer: C tokens per sequence in one call.
//
// Definition: the result equals C successive (append, decode) steps -- each token
// is appended to the window ring and the pending block and then attends, with the
// same readings as the single-token path (fluxbbs.com "EdgeRock-4B 开源：72 MiB 固定
// KV…", section "架构：递归、局部窗口与记忆锚点三件套": learned RMS norm and rotary on
// q and k, 16 query heads over 4 KV groups; neodrop.ai repost "内存还会跌吗？…",
// section "三段记忆，只记值得记的": one candidate per token into the pending block).
// Token i of sequence b sits at position p0 + 1 + i with p0 = pos[b]; it sees the
// window positions p - 1023 .. p, all committed anchors, and the pending records
// at positions <= p.
//
// Three launches:
//  1. prefill_write: normalise + rotate the chunk's keys; the anchor candidates go
//     straight into pending rows n_pend .. n_pend + C - 1, the window keys into the
//     workspace (the ring cannot be overwritten yet: earlier tokens of the chunk
//     still read the positions the chunk will replace).
//  2. prefill_attn: one workgroup per (branch, sequence, group, 16-token tile): 64
//     query rows (16 tokens x 4 heads), 16 per wave.  Key tiles of 16 are staged
//     once in LDS for the four waves -- K row-major, V transposed -- and every key
//     is masked by its position.  S^T = K Q^T and O^T += V^T P^T on MFMA, as in the
//     decode kernel; the tiles of one unit are numbered onto one XCD so they share
//     its L2.
//  3. prefill_ring: copy the chunk's window K/V into ring slots, then advance
//     n_pend and pos.
#include "rma_device.h"

namespace rma {

constexpr int kPTok = 16;                          // tokens per attention workgroup
constexpr int kPRowsWave = 16;                     // query rows per wave (4 tokens x 4 heads)
constexpr int kPWaves = kPTok * kHeadsPerGroup / kPRowsWave;  // 4
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPKeys = 16;                         // keys per tile
constexpr int kKStr = kDim + 8;                    // K tile row stride (elements)
constexpr int kVtStr = kPKeys + 8;                 // V^T tile row stride (elements)
constexpr int kMaxChunk = kBlock;
constexpr float kPQScale = 1.4426950408889634f / 16.0f;
constexpr float kPLn2 = 0.69314718055994531f;
constexpr int kXcds = 8;

template <typename T, typename F>
__device__ __forceinline__ T pbitcast(const F &f) {
  return __builtin_bit_cast(T, f);
}

struct PrefillParams {
  uint16_t *win_k, *win_v, *bank_k, *bank_v, *pend_k, *pend_v;
  float *pend_score;
  int32_t *pend_src, *n_bank, *n_pend, *pos;
  const uint16_t *k_win, *v_win, *k_rma, *v_rma;  // [B][C][4][256]
  const float *score;                             // [B][C][4] or null
  const uint16_t *q_win, *q_rma;                  // [B][C][16][256]
  const float *gq_win, *gk_win, *gq_rma, *gk_rma;
  float eps;
  double rope_ratio;
  uint16_t *o_win, *o_rma;  // [B][C][16][256]
  float *lse_win, *lse_rma; // [B][C][16]
  uint16_t *wk;             // workspace: chunk window keys [B][C][4][256]
  int batch, chunk;
};

__device__ __forceinline__ bool chunk_fits(const PrefillParams &a, int b) {
  const int np = a.n_pend[b];
  return np >= 0 && np + a.chunk <= kBlock;
}

// ---------------------------------------------------------------- 1. write
__global__ __launch_bounds__(256) void prefill_write_kernel(PrefillParams a) {
  const int b = blockIdx.x / a.chunk;
  const int i = blockIdx.x % a.chunk;
  const int g = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  if (!chunk_fits(a, b)) return;
  const int np0 = a.n_pend[b];
  const int p = a.pos[b] + 1 + i;
  const size_t in = ((static_cast<size_t>(b) * a.chunk + i) * kGroups + g) * kDim + 4 * lane;
  const size_t prow = ((static_cast<size_t>(b) * kGroups + g) * kBlock + np0 + i) * kDim + 4 * lane;
  const uint2 kw = *reinterpret_cast<const uint2 *>(a.k_win + in);
  const uint2 kr = *reinterpret_cast<const uint2 *>(a.k_rma + in);
  float xw[4] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y)};
  float xr[4] = {bf16_lo(kr.x), bf16_hi(kr.x), bf16_lo(kr.y), bf16_hi(kr.y)};
  float c, sn;
  rope_cos_sin(a.rope_ratio, p, lane, c, sn);
  norm_rope_head(xw, a.gk_win, a.eps, c, sn, lane);
  norm_rope_head(xr, a.gk_rma, a.eps, c, sn, lane);
  *reinterpret_cast<uint2 *>(a.wk + in) =
      make_uint2(pack_bf16x2(xw[0], xw[1]), pack_bf16x2(xw[2], xw[3]));
  *reinterpret_cast<uint2 *>(a.pend_k + prow) =
      make_uint2(pack_bf16x2(xr[0], xr[1]), pack_bf16x2(xr[2], xr[3]));
  *reinterpret_cast<uint2 *>(a.pend_v + prow) = *reinterpret_cast<const uint2 *>(a.v_rma + in);
  if (lane == 0) {
    if (a.score)
      a.pend_score[(static_cast<size_t>(b) * kBlock + np0 + i) * kGroups + g] =
          a.score[(static_cast<size_t>(b) * a.chunk + i) * kGroups + g];
    if (g == 0) a.pend_src[static_cast<size_t>(b) * kBlock + np0 + i] = p;
  }
}

// ---------------------------------------------------------------- 2. attention
// A run of key rows and how each row's position is known.
struct PSeg {
  const uint16_t *k, *v;  // row-major, 256 BF16 per row
  int n;                  // rows
  int kind;               // 0: always visible; 1: window ring slot; 2: chunk row
};

__global__ __launch_bounds__(kPThreads, 2) void prefill_attn_kernel(PrefillParams a) {
  __shared__ __align__(16) uint16_t q_lds[kPTok * kHeadsPerGroup][kDim];
  __shared__ __align__(16) uint16_t k_lds[2][kPKeys * kKStr];
  __shared__ __align__(16) uint16_t vt_lds[2][kDim * kVtStr];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const int ntile = (a.chunk + kPTok - 1) / kPTok;
  // XCD-aware numbering: the tiles of one unit run on one XCD, one after another.
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds, slot = bid / kXcds;
  const int unit = (slot / ntile) * kXcds + xcd;
  const int tt = slot % ntile;
  const int nunits = a.batch * kGroups * 2;
  if (unit >= nunits) return;
  const bool anchor = unit < a.batch * kGroups;
  const int bg = anchor ? unit : unit - a.batch * kGroups;
  const int b = bg / kGroups, g = bg % kGroups;
  const int tok0 = tt * kPTok;
  const int ntok = min(kPTok, a.chunk - tok0);
  const size_t sgi = static_cast<size_t>(b) * kGroups + g;

  const bool fits = chunk_fits(a, b);
  const int p0 = a.pos[b];  // position before the chunk
  const int np0 = fits ? a.n_pend[b] : 0;

  // segments of this branch (named, not indexed, so they stay in scalar registers)
  PSeg seg0, seg1, seg2;
  if (anchor) {
    const int nb = min(max(a.n_bank[b], 0), kBank);
    seg0 = {a.bank_k + sgi * kBank * kDim, a.bank_v + sgi * kBank * kDim, nb, 0};
    seg1 = {a.pend_k + sgi * kBlock * kDim, a.pend_v + sgi * kBlock * kDim, np0, 0};
    seg2 = {a.pend_k + (sgi * kBlock + np0) * kDim, a.pend_v + (sgi * kBlock + np0) * kDim,
            tok0 + ntok, 2};
  } else {
    const int nw = min(max(p0 + 1, 0), kWindow);
    seg0 = {a.win_k + sgi * kWindow * kDim, a.win_v + sgi * kWindow * kDim, nw, 1};
    seg1 = {nullptr, nullptr, 0, 0};
    // chunk window rows: keys from the workspace, values straight from the input
    seg2 = {a.wk + static_cast<size_t>(b) * a.chunk * kGroups * kDim + g * kDim,
            a.v_win + static_cast<size_t>(b) * a.chunk * kGroups * kDim + g * kDim,
            tok0 + ntok, 2};
  }
  // (chunk rows are strided by the 4 groups of the [C][4][256] workspace/input layout)

  // ---- query prep: wave w owns rows 16w .. 16w+15 = tokens 4w .. 4w+3, heads 0..3
  for (int r = 0; r < kPRowsWave; ++r) {
    const int row = wave * kPRowsWave + r;
    const int tl = row / kHeadsPerGroup, h = row % kHeadsPerGroup;
    uint2 o = make_uint2(0, 0);
    if (tl < ntok && fits) {
      const int tok = tok0 + tl;
      const uint16_t *q = (anchor ? a.q_rma : a.q_win) +
                          ((static_cast<size_t>(b) * a.chunk + tok) * kHeads + g * kHeadsPerGroup + h) * kDim;
      const uint2 raw = *reinterpret_cast<const uint2 *>(q + 4 * lane);
      float x[4] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y)};
      float c, sn;
      rope_cos_sin(a.rope_ratio, p0 + 1 + tok, lane, c, sn);
      norm_rope_head(x, anchor ? a.gq_rma : a.gq_win, a.eps, c, sn, lane);
      o.x = pack_bf16x2(x[0] * kPQScale, x[1] * kPQScale);
      o.y = pack_bf16x2(x[2] * kPQScale, x[3] * kPQScale);
    }
    *reinterpret_cast<uint2 *>(&q_lds[row][4 * lane]) = o;
  }
  __syncthreads();
  const int rl = lane & 15, kg = lane >> 4;  // lane's query row (within the wave) and key group
  bf16x8 qb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qb[s] = pbitcast<bf16x8>(
        *reinterpret_cast<const uint4 *>(&q_lds[wave * kPRowsWave + rl][32 * s + 8 * kg]));
  // this lane's query token and its position
  const int my_tl = (wave * kPRowsWave + rl) / kHeadsPerGroup;
  const int my_tok = tok0 + my_tl;
  const int my_pos = p0 + 1 + my_tok;
  const bool my_row_ok = my_tl < ntok && fits;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  // staging role: key (tid / 16), dims 16 * (tid % 16) .. +16
  const int sk = tid >> 4, sd = (tid & 15) * 16;

  // tile list: segment s contributes ceil(n / 16) tiles; chunk tiles past this
  // workgroup's last token are invisible to all its rows and are not in the list
  const int tl0 = (seg0.n + kPKeys - 1) / kPKeys;
  const int tl1 = (seg1.n + kPKeys - 1) / kPKeys;
  const int tl2 = (seg2.n + kPKeys - 1) / kPKeys;
  const int total = tl0 + tl1 + tl2;
  const size_t stride2 = anchor ? kDim : static_cast<size_t>(kGroups) * kDim;

  // Global -> registers for tile t (all values wave-uniform except the lane offset).
  uint4 kr0, kr1, vr0, vr1;
#define PREFILL_LOAD_TILE(t_)                                                                 \
  {                                                                                           \
    const int t__ = (t_);                                                                     \
    const int si = t__ < tl0 ? 0 : (t__ < tl0 + tl1 ? 1 : 2);                                 \
    const int key = (t__ - (si == 0 ? 0 : (si == 1 ? tl0 : tl0 + tl1))) * kPKeys + sk;        \
    const uint16_t *kb = si == 0 ? seg0.k : (si == 1 ? seg1.k : seg2.k);                      \
    const uint16_t *vb = si == 0 ? seg0.v : (si == 1 ? seg1.v : seg2.v);                      \
    const int n = si == 0 ? seg0.n : (si == 1 ? seg1.n : seg2.n);                             \
    const size_t st = si == 2 ? stride2 : static_cast<size_t>(kDim);                          \
    kr0 = kr1 = vr0 = vr1 = make_uint4(0, 0, 0, 0);                                           \
    if (key < n) {                                                                            \
      const uint4 *kp = reinterpret_cast<const uint4 *>(kb + static_cast<size_t>(key) * st + sd); \
      const uint4 *vp = reinterpret_cast<const uint4 *>(vb + static_cast<size_t>(key) * st + sd); \
      kr0 = kp[0];                                                                            \
      kr1 = kp[1];                                                                            \
      vr0 = vp[0];                                                                            \
      vr1 = vp[1];                                                                            \
    }                                                                                         \
  }
  // Registers -> LDS buffer buf: K row-major, V transposed (V^T[dim][key]).
#define PREFILL_STORE_TILE(buf_)                                                              \
  {                                                                                           \
    uint4 *kd = reinterpret_cast<uint4 *>(&k_lds[(buf_)][sk * kKStr + sd]);                   \
    kd[0] = kr0;                                                                              \
    kd[1] = kr1;                                                                              \
    uint16_t *vt = &vt_lds[(buf_)][sd * kVtStr + sk];                                         \
    const uint32_t w0 = vr0.x, w1 = vr0.y, w2 = vr0.z, w3 = vr0.w;                            \
    const uint32_t w4 = vr1.x, w5 = vr1.y, w6 = vr1.z, w7 = vr1.w;                            \
    vt[0 * kVtStr] = w0 & 0xffffu;  vt[1 * kVtStr] = w0 >> 16;                                \
    vt[2 * kVtStr] = w1 & 0xffffu;  vt[3 * kVtStr] = w1 >> 16;                                \
    vt[4 * kVtStr] = w2 & 0xffffu;  vt[5 * kVtStr] = w2 >> 16;                                \
    vt[6 * kVtStr] = w3 & 0xffffu;  vt[7 * kVtStr] = w3 >> 16;                                \
    vt[8 * kVtStr] = w4 & 0xffffu;  vt[9 * kVtStr] = w4 >> 16;                                \
    vt[10 * kVtStr] = w5 & 0xffffu; vt[11 * kVtStr] = w5 >> 16;                               \
    vt[12 * kVtStr] = w6 & 0xffffu; vt[13 * kVtStr] = w6 >> 16;                               \
    vt[14 * kVtStr] = w7 & 0xffffu; vt[15 * kVtStr] = w7 >> 16;                               \
  }

  if (total > 0) {
    PREFILL_LOAD_TILE(0);
    PREFILL_STORE_TILE(0);
  }
  __syncthreads();
  for (int t = 0; t < total; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < total;
    if (more) PREFILL_LOAD_TILE(t + 1);
    const int si = t < tl0 ? 0 : (t < tl0 + tl1 ? 1 : 2);
    const int ck0 = (t - (si == 0 ? 0 : (si == 1 ? tl0 : tl0 + tl1))) * kPKeys;
    const int cn = si == 0 ? seg0.n : (si == 1 ? seg1.n : seg2.n);
    const int ckind = si == 0 ? seg0.kind : (si == 1 ? seg1.kind : seg2.kind);
    // S^T = K Q^T: lane holds keys 4kg+i (i = 0..3) of row rl
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t *krow = &k_lds[buf][rl * kKStr + 8 * kg];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 kv = pbitcast<bf16x8>(*reinterpret_cast<const uint4 *>(krow + 32 * s));
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[s], sc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = ck0 + 4 * kg + i;
      bool vis = my_row_ok && key < cn;
      if (ckind == 1) {
        const int kp = p0 - ((p0 - key) & (kWindow - 1));
        vis = vis && kp >= 0 && kp >= my_pos - (kWindow - 1);
      } else if (ckind == 2) {
        vis = vis && key <= my_tok;
      }
      if (!vis) sc[i] = -INFINITY;
    }
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    float alpha = 1.f;
    uint32_t pw0 = 0, pw1 = 0;
    float psum = 0.f;
    if (m_new != -INFINITY) {
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      const uint32_t q0 = f32_to_bf16(__builtin_amdgcn_exp2f(sc[0] - m_new));
      const uint32_t q1 = f32_to_bf16(__builtin_amdgcn_exp2f(sc[1] - m_new));
      const uint32_t q2 = f32_to_bf16(__builtin_amdgcn_exp2f(sc[2] - m_new));
      const uint32_t q3 = f32_to_bf16(__builtin_amdgcn_exp2f(sc[3] - m_new));
      psum = (bf16_to_f32(q0) + bf16_to_f32(q1)) + (bf16_to_f32(q2) + bf16_to_f32(q3));
      pw0 = q0 | (q1 << 16);
      pw1 = q2 | (q3 << 16);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const s16x4 pb = pbitcast<s16x4>(make_uint2(pw0, pw1));
    // O^T += V^T P^T: lane holds dims 16db + 4kg + i of row rl
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const uint2 w = *reinterpret_cast<const uint2 *>(&vt_lds[buf][(db * 16 + rl) * kVtStr + 4 * kg]);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pbitcast<s16x4>(w), pb, acc[db] * alpha,
                                                          0, 0, 0);
    }
    if (more) PREFILL_STORE_TILE(buf ^ 1);
    __syncthreads();
  }
#undef PREFILL_LOAD_TILE
#undef PREFILL_STORE_TILE

  // epilogue: row rl of this wave = token my_tok, head h
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const int h = (wave * kPRowsWave + rl) % kHeadsPerGroup;
  const int head = g * kHeadsPerGroup + h;
  if (my_tl < ntok) {
    uint16_t *o = (anchor ? a.o_rma : a.o_win) +
                  ((static_cast<size_t>(b) * a.chunk + my_tok) * kHeads + head) * kDim;
    const bool empty = m_run == -INFINITY;
    const float inv = empty ? 0.f : 1.f / l_tot;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      uint2 ov = make_uint2(0, 0);
      if (!empty) {
        ov.x = pack_bf16x2(acc[db][0] * inv, acc[db][1] * inv);
        ov.y = pack_bf16x2(acc[db][2] * inv, acc[db][3] * inv);
      }
      *reinterpret_cast<uint2 *>(o + db * 16 + 4 * kg) = ov;
    }
    if (kg == 0) {
      float *lse = (anchor ? a.lse_rma : a.lse_win) +
                   (static_cast<size_t>(b) * a.chunk + my_tok) * kHeads + head;
      *lse = empty ? -INFINITY : (m_run + log2f(l_tot)) * kPLn2;
    }
  }
}

// ---------------------------------------------------------------- 3. ring + counters
__global__ __launch_bounds__(256) void prefill_ring_kernel(PrefillParams a) {
  const int b = blockIdx.x / a.chunk;
  const int i = blockIdx.x % a.chunk;
  const int g = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  if (!chunk_fits(a, b)) return;
  const int p = a.pos[b] + 1 + i;
  const size_t in = ((static_cast<size_t>(b) * a.chunk + i) * kGroups + g) * kDim + 4 * lane;
  const size_t w_row =
      ((static_cast<size_t>(b) * kGroups + g) * kWindow + (p & (kWindow - 1))) * kDim + 4 * lane;
  *reinterpret_cast<uint2 *>(a.win_k + w_row) = *reinterpret_cast<const uint2 *>(a.wk + in);
  *reinterpret_cast<uint2 *>(a.win_v + w_row) = *reinterpret_cast<const uint2 *>(a.v_win + in);
}

__global__ __launch_bounds__(256) void prefill_counters_kernel(PrefillParams a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.batch || !chunk_fits(a, b)) return;
  a.n_pend[b] += a.chunk;
  a.pos[b] += a.chunk;
}

}  // namespace rma

using namespace rma;

static bool pf_aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

extern "C" size_t rma_prefill_workspace_bytes(int32_t batch, int32_t n_tokens) {
  if (batch <= 0 || n_tokens <= 0) return 0;
  return static_cast<size_t>(batch) * n_tokens * kGroups * kDim * sizeof(uint16_t);
}

extern "C" rma_status swa_rma_prefill(const rma_layer_state *st, int32_t batch, int32_t n_tokens,
                                      const uint16_t *k_win, const uint16_t *v_win,
                                      const uint16_t *k_rma, const uint16_t *v_rma,
                                      const float *score, const uint16_t *q_win,
                                      const uint16_t *q_rma, const rma_norm *norm,
                                      uint16_t *o_win, float *lse_win, uint16_t *o_rma,
                                      float *lse_rma, void *workspace, size_t workspace_bytes,
                                      void *stream) {
  if (!st || !norm || !k_win || !v_win || !k_rma || !v_rma || !q_win || !q_rma || !o_win ||
      !lse_win || !o_rma || !lse_rma)
    return RMA_E_ARG;
  if (batch <= 0 || batch > RMA_MAX_BATCH || n_tokens <= 0 || n_tokens > kMaxChunk)
    return RMA_E_ARG;
  if (!st->win_k || !st->win_v || !st->bank_k || !st->bank_v || !st->pend_k || !st->pend_v ||
      !st->pend_src || !st->n_bank || !st->n_pend || !st->pos || !norm->gq_win ||
      !norm->gk_win || !norm->gq_rma || !norm->gk_rma || (score && !st->pend_score))
    return RMA_E_ARG;
  const void *al[] = {st->win_k, st->win_v, st->bank_k, st->bank_v, st->pend_k, st->pend_v,
                      k_win,     v_win,     k_rma,      v_rma,      q_win,      q_rma,
                      o_win,     o_rma,     norm->gq_win, norm->gk_win, norm->gq_rma,
                      norm->gk_rma};
  for (const void *p : al)
    if (!pf_aligned16(p)) return RMA_E_ALIGN;
  const size_t need = rma_prefill_workspace_bytes(batch, n_tokens);
  if (!workspace || workspace_bytes < need) return RMA_E_WORKSPACE;
  if (!pf_aligned16(workspace)) return RMA_E_ALIGN;

  PrefillParams p;
  p.win_k = st->win_k;
  p.win_v = st->win_v;
  p.bank_k = st->bank_k;
  p.bank_v = st->bank_v;
  p.pend_k = st->pend_k;
  p.pend_v = st->pend_v;
  p.pend_score = st->pend_score;
  p.pend_src = st->pend_src;
  p.n_bank = st->n_bank;
  p.n_pend = st->n_pend;
  p.pos = st->pos;
  p.k_win = k_win;
  p.v_win = v_win;
  p.k_rma = k_rma;
  p.v_rma = v_rma;
  p.score = score;
  p.q_win = q_win;
  p.q_rma = q_rma;
  p.gq_win = norm->gq_win;
  p.gk_win = norm->gk_win;
  p.gq_rma = norm->gq_rma;
  p.gk_rma = norm->gk_rma;
  p.eps = norm->eps;
  p.rope_ratio = rope_ratio(norm->rope_base);
  p.o_win = o_win;
  p.o_rma = o_rma;
  p.lse_win = lse_win;
  p.lse_rma = lse_rma;
  p.wk = static_cast<uint16_t *>(workspace);
  p.batch = batch;
  p.chunk = n_tokens;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned rows = static_cast<unsigned>(batch) * static_cast<unsigned>(n_tokens);
  hipLaunchKernelGGL(prefill_write_kernel, dim3(rows), dim3(256), 0, s, p);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  const unsigned ntile = (n_tokens + kPTok - 1) / kPTok;
  const unsigned units = static_cast<unsigned>(batch) * kGroups * 2;
  // units padded to a multiple of the XCD count so every XCD slot maps to a unit
  const unsigned units_pad = (units + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3(units_pad * ntile), dim3(kPThreads), 0, s, p);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  hipLaunchKernelGGL(prefill_ring_kernel, dim3(rows), dim3(256), 0, s, p);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  hipLaunchKernelGGL(prefill_counters_kernel, dim3((batch + 255) / 256), dim3(256), 0, s, p);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  return RMA_OK;
}
