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
//  2. prefill_attn: one workgroup per (branch, sequence, group, 64-token tile): 256
//     query rows (64 tokens x 4 heads), 32 per wave, eight waves (two per SIMD),
//     held in VGPRs in the operand layout of v_mfma_f32_32x32x16_bf16 after norm +
//     rotary.  Every K/V tile brought into LDS serves 256 rows: the L2-to-LDS
//     traffic per flop is half that of 128-row workgroups, and that traffic ran
//     close to the MFMA time.  Key tiles of 32 reach LDS through buffer loads
//     straight into LDS, four stages deep (three tiles in flight while one is
//     computed); rows are XOR-swizzled against bank conflicts.  S^T = K Q^T reads
//     K rows; O^T += V^T P^T reads V^T with transposing LDS reads, in the key
//     order of the score accumulator, so P goes from registers straight into the
//     second product.  Keys are masked by position (ring age, causal order in the
//     chunk).  The softmax reference maximum moves only when a row's maximum grows
//     by more than 2^8, so the 128 accumulators are rarely rescaled.  The rotary
//     (cos, sin) of each (token, pair) is formed once per wave and shared across
//     the token's four heads.  The tiles of one unit are numbered onto one XCD so
//     they share its L2.
//  3. prefill_ring: copy the chunk's window K/V into ring slots, then advance
//     n_pend and pos.
#include "rma_device.h"

namespace rma {

constexpr int kPWaves = 8;                         // waves per attention workgroup (2 per SIMD)
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPRowsWave = 32;                     // query rows per wave (8 tokens x 4 heads)
constexpr int kPTok = kPWaves * kPRowsWave / kHeadsPerGroup;  // 64 tokens per workgroup
constexpr int kPKeys = 32;                         // keys per tile
constexpr int kStages = 4;                         // LDS tile buffers (3 tiles in flight)
constexpr int kTileElems = kPKeys * kDim;          // one K or V tile, row-major, 16 KB
constexpr int kDmaPerTile = 2 * kTileElems * 2 / (kPThreads * 16);  // per wave: 8
constexpr int kMaxChunk = kBlock;
constexpr float kPQScale = 1.4426950408889634f / 16.0f;
constexpr float kPLn2 = 0.69314718055994531f;
constexpr float kPTau = 8.0f;  // reference-maximum slack (log2 units): P <= 2^8
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
// A run of key rows and how each row's position is known.  K and V are read
// through buffer resources whose range ends at the last row, so rows past the
// end read as zero.
struct PSeg {
  __amdgpu_buffer_rsrc_t k, v;
  int n;       // rows
  int stride;  // bytes between rows
  int kind;    // 0: always visible; 1: window ring slot; 2: chunk row
};

__device__ __forceinline__ PSeg make_pseg(const uint16_t *k, const uint16_t *v, int n,
                                          int stride_elems, int kind) {
  const int bytes = n > 0 ? (n - 1) * stride_elems * 2 + kDim * 2 : 0;
  PSeg sg;
  sg.k = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(k), 0, bytes, 0x00020000);
  sg.v = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(v), 0, bytes, 0x00020000);
  sg.n = n;
  sg.stride = stride_elems * 2;
  sg.kind = kind;
  return sg;
}

__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// LDS tile layouts, chosen so that the MFMA operand reads below spread over all
// banks (gfx950 LDS serves 256 bytes per clock: 16 lanes of a 16-byte read, 32
// lanes of an 8-byte transposed read):
//  * K: key pair j (keys j and j + 16, 512 bytes each) at byte 1040 j, the 16
//    bytes after each pair unused.  Lanes 0..15 of a read take keys 0..15 at one
//    chunk: 1040 j is 16 j modulo 256, so the 16 reads cover the 64 banks once.
//    A lane's reads of a tile then differ only by immediate offsets (one address
//    register), and one load-to-LDS instruction (64 lanes x 16 bytes) fills one
//    pair, each half-wave reading 512 contiguous bytes of one key.
//  * V: row-major, chunk c of key k at chunk position c ^ (4 (k & 3)).
constexpr int kKPairBytes = 2 * kDim * 2 + 16;                  // 1040
constexpr int kKStageElems = kPKeys / 2 * kKPairBytes / 2;      // 8320 (16,640 bytes)
__device__ __forceinline__ int v_swz(int key) { return 4 * (key & 3); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
constexpr uint32_t kOnesBf16x2Bits = 0x3f803f80u;  // (1.0, 1.0) in BF16
#define kOnesBf16x2 pbitcast<bf16x2_t>(kOnesBf16x2Bits)
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

// Wait until this wave has at most N vector-memory operations in flight, then
// meet the other waves at the barrier.  (A plain __syncthreads() would also wait
// for every outstanding load-to-LDS, i.e. for the tiles still meant to be in flight.)
// One K and one V tile buffer per pipeline stage, as separate arrays so that the
// compiler's wait for loads-to-LDS can tell the stage being read from the stages
// still being filled.
__shared__ __align__(16) uint16_t pf_k0[kKStageElems];
__shared__ __align__(16) uint16_t pf_k1[kKStageElems];
__shared__ __align__(16) uint16_t pf_k2[kKStageElems];
__shared__ __align__(16) uint16_t pf_k3[kKStageElems];
__shared__ __align__(16) uint16_t pf_v0[kTileElems];
__shared__ __align__(16) uint16_t pf_v1[kTileElems];
__shared__ __align__(16) uint16_t pf_v2[kTileElems];
__shared__ __align__(16) uint16_t pf_v3[kTileElems];
static_assert(kStages == 4, "the tile loop below is written out for four stages");
// Per-thread LDS offsets, read back per tile (keeping them in registers across the
// tile loop would cost registers the loop needs): the lane's V chunk offsets of
// its two V loads, and its four V^T read offsets.
typedef int pf_i32x4 __attribute__((ext_vector_type(4)));
typedef volatile __attribute__((address_space(3))) pf_i32x4 lds_vi32x4;
__shared__ pf_i32x4 pf_dma_tab[kPThreads];
__shared__ pf_i32x4 pf_vrd_tab[kPThreads];

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

__global__ __launch_bounds__(kPThreads) void prefill_attn_kernel(PrefillParams a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps per-wave tests scalar
  const int ntile = (a.chunk + kPTok - 1) / kPTok;
  // XCD-aware numbering: the token tiles of one unit run on one XCD.
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
  const int nchunk = fits ? min(tok0 + kPTok, a.chunk) : 0;  // chunk keys any row here sees
  PSeg seg0, seg1, seg2;
  if (anchor) {
    const int nb = fits ? min(max(a.n_bank[b], 0), kBank) : 0;
    seg0 = make_pseg(a.bank_k + sgi * kBank * kDim, a.bank_v + sgi * kBank * kDim, nb, kDim, 0);
    seg1 = make_pseg(a.pend_k + sgi * kBlock * kDim, a.pend_v + sgi * kBlock * kDim, np0, kDim, 0);
    seg2 = make_pseg(a.pend_k + (sgi * kBlock + np0) * kDim,
                     a.pend_v + (sgi * kBlock + np0) * kDim, nchunk, kDim, 2);
  } else {
    const int nw = fits ? min(max(p0 + 1, 0), kWindow) : 0;
    seg0 = make_pseg(a.win_k + sgi * kWindow * kDim, a.win_v + sgi * kWindow * kDim, nw, kDim, 1);
    seg1 = seg0;
    seg1.n = 0;
    // chunk window rows: keys from the workspace, values straight from the input,
    // both in the [C][4][256] layout (rows strided by the 4 groups)
    seg2 = make_pseg(a.wk + static_cast<size_t>(b) * a.chunk * kGroups * kDim + g * kDim,
                     a.v_win + static_cast<size_t>(b) * a.chunk * kGroups * kDim + g * kDim,
                     nchunk, kGroups * kDim, 2);
  }

  // tile list: segment s contributes ceil(n / 32) tiles
  const int tl0 = (seg0.n + kPKeys - 1) / kPKeys;
  const int tl1 = (seg1.n + kPKeys - 1) / kPKeys;
  const int tl2 = (seg2.n + kPKeys - 1) / kPKeys;
  const int total = tl0 + tl1 + tl2;

#define PREFILL_TILE_SEG(t_, sg_, k0_)                                                       \
  const int si_##sg_ = (t_) < tl0 ? 0 : ((t_) < tl0 + tl1 ? 1 : 2);                          \
  const PSeg &sg_ = si_##sg_ == 0 ? seg0 : (si_##sg_ == 1 ? seg1 : seg2);                    \
  const int k0_ = ((t_) - (si_##sg_ == 0 ? 0 : (si_##sg_ == 1 ? tl0 : tl0 + tl1))) * kPKeys;

  // Load-to-LDS of tile t into stage st: each wave moves 2 KB of K and 2 KB of V,
  // 1 KB per instruction.  K: the instruction for key pair j fills its 1040-byte
  // slot, lane L taking chunk L % 32 of key j + 16 (L / 32).  V: lane L fills chunk
  // position L % 32 of row 2i + L / 32, i.e. fetches the chunk that the swizzle
  // puts there.  Rows past the segment's end read as zero.
  // The tile's first row and the wave's row pair go into the scalar offset; the
  // lane's part of a V load (odd row of the pair, swizzled chunk) is fixed per
  // load, formed once here and kept in an LDS table that each tile reads back.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  constexpr int kPairs = kPKeys / 2 / kPWaves;  // row pairs each wave moves per tile: 2
  static_assert(kPairs == 2, "the offset table holds two K and two V chunk offsets");
  {
    const int rlo = lane >> 5, cpos = lane & 31;
    pf_i32x4 t;
    const int row0 = 2 * (kPairs * wave_s) + rlo, row1 = row0 + 2;
    t.x = 0;
    t.y = 0;
    t.z = (cpos ^ v_swz(row0)) << 4;
    t.w = (cpos ^ v_swz(row1)) << 4;
    pf_dma_tab[threadIdx.x] = t;
  }
#define PREFILL_ISSUE_TILE(t_, kdst_, vdst_)                                                 \
  {                                                                                          \
    PREFILL_TILE_SEG(t_, isg, ik0)                                                           \
    const pf_i32x4 dt = ((lds_vi32x4 *)pf_dma_tab)[threadIdx.x];                             \
    const int lo_off = (lane >> 5) * isg.stride;                                             \
    const int k_off = 16 * lo_off + ((lane & 31) << 4);                                      \
    const int vc[2] = {dt.z, dt.w};                                                          \
    _Pragma("unroll") for (int i = 0; i < kPairs; ++i) {                                     \
      const int pr = kPairs * wave_s + i;                                                    \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                              \
          isg.k, (lds_void *)(reinterpret_cast<char *>(kdst_) + pr * kKPairBytes), 16, k_off, \
          (ik0 + pr) * isg.stride, 0, 0);                                                    \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isg.v, (lds_void *)&vdst_[pr * 2 * kDim], 16, \
                                               lo_off + vc[i], (ik0 + 2 * pr) * isg.stride,  \
                                               0, 0);                                        \
    }                                                                                        \
  }
  // Start the first tiles' loads before the query prologue.
  if (total > 0) PREFILL_ISSUE_TILE(0, pf_k0, pf_v0);
  if (total > 1) PREFILL_ISSUE_TILE(1, pf_k1, pf_v1);
  if (total > 2) PREFILL_ISSUE_TILE(2, pf_k2, pf_v2);

  // ---- query: lane l holds row rl = l % 32 of this wave (token 8w + rl/4, head
  // rl % 4), dims 16s + 8hh .. +7 for s = 0..15 -- the B operand layout of
  // v_mfma_f32_32x32x16_bf16.  Normalised, rotated and scaled by log2(e)/16 here.
  const int rl = lane & 31, hh = lane >> 5;
  const int my_tl = wave * (kPRowsWave / kHeadsPerGroup) + rl / kHeadsPerGroup;
  const int my_head = rl % kHeadsPerGroup;
  const int my_tok = tok0 + my_tl;
  const bool my_row_ok = my_tl < ntok && fits;
  bf16x8 qb[16];
  {
    const uint16_t *qrow =
        (anchor ? a.q_rma : a.q_win) +
        ((static_cast<size_t>(b) * a.chunk + min(my_tok, a.chunk - 1)) * kHeads +
         g * kHeadsPerGroup + my_head) * kDim + 8 * hh;
    const float *gam = (anchor ? a.gq_rma : a.gq_win) + 8 * hh;
    u32x4 raw[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) raw[s] = *reinterpret_cast<const u32x4 *>(qrow + 16 * s);
    // (cos, sin) of the wave's 8 tokens x 32 rotary pairs, each formed once: lane L
    // takes token L / 8 and pairs 4 (L % 8) .. +3 (theta_i = r^i by binary powering
    // for the first pair, then repeated multiplication)
    float rc[4], rsn[4];
    {
      const int tpos = p0 + 1 + tok0 + wave * (kPRowsWave / kHeadsPerGroup) + (lane >> 3);
      const int i0 = 4 * (lane & 7);
      double theta = 1.0, sq = a.rope_ratio;
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        if ((i0 >> k) & 1) theta *= sq;
        sq *= sq;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rope_cos_sin_theta(theta, tpos, rc[j], rsn[j]);
        theta *= a.rope_ratio;
      }
    }
    float ssp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_lo(raw[s][e]), hi = bf16_hi(raw[s][e]);
        ssp[e] = fmaf(lo, lo, fmaf(hi, hi, ssp[e]));
      }
    float ss = (ssp[0] + ssp[1]) + (ssp[2] + ssp[3]);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = 1.0f / sqrtf(ss * (1.0f / kDim) + a.eps);
    const float inv_sc = my_row_ok ? inv * kPQScale : 0.f;  // rows not stored get zeros
    // dims past the rotary part: scale and pack in place
#pragma unroll
    for (int s = 4; s < 16; ++s) {
      const float4 g0 = *reinterpret_cast<const float4 *>(gam + 16 * s);
      const float4 g1 = *reinterpret_cast<const float4 *>(gam + 16 * s + 4);
      const float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = pack_bf16x2_hw(bf16_lo(raw[s][e]) * inv_sc * gm[2 * e],
                              bf16_hi(raw[s][e]) * inv_sc * gm[2 * e + 1]);
      qb[s] = pbitcast<bf16x8>(w);
    }
    // rotary dims i = 16s + 8hh + e (s = 0, 1) pair with i + 32 (chunk s + 2, same
    // lane); their (cos, sin) sit in lane 8 (rl / 4) + i / 4, slot i % 4
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float4 ga0 = *reinterpret_cast<const float4 *>(gam + 16 * s);
      const float4 ga1 = *reinterpret_cast<const float4 *>(gam + 16 * s + 4);
      const float4 gb0 = *reinterpret_cast<const float4 *>(gam + 16 * (s + 2));
      const float4 gb1 = *reinterpret_cast<const float4 *>(gam + 16 * (s + 2) + 4);
      const float gma[8] = {ga0.x, ga0.y, ga0.z, ga0.w, ga1.x, ga1.y, ga1.z, ga1.w};
      const float gmb[8] = {gb0.x, gb0.y, gb0.z, gb0.w, gb1.x, gb1.y, gb1.z, gb1.w};
      float y1[8], y2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int src = 8 * (rl >> 2) + 4 * s + 2 * hh + (e >> 2);
        const float c = __shfl(rc[e & 3], src, 64);
        const float sn = __shfl(rsn[e & 3], src, 64);
        const uint32_t ra = raw[s][e >> 1], rb = raw[s + 2][e >> 1];
        const float x1 = ((e & 1) ? bf16_hi(ra) : bf16_lo(ra)) * inv * gma[e];
        const float x2 = ((e & 1) ? bf16_hi(rb) : bf16_lo(rb)) * inv * gmb[e];
        const float k = my_row_ok ? kPQScale : 0.f;
        y1[e] = (x1 * c - x2 * sn) * k;
        y2[e] = (x2 * c + x1 * sn) * k;
      }
      u32x4 wa, wb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wa[e] = pack_bf16x2_hw(y1[2 * e], y1[2 * e + 1]);
        wb[e] = pack_bf16x2_hw(y2[2 * e], y2[2 * e + 1]);
      }
      qb[s] = pbitcast<bf16x8>(wa);
      qb[s + 2] = pbitcast<bf16x8>(wb);
    }
  }
  // The query operands stay in VGPRs: with two waves per SIMD a wave has 256
  // registers, and any AGPR use would split them evenly between the two files,
  // while the tile loop needs about 250 arch VGPRs (128 accumulators, 64 query
  // operands, scores, operand reads and LDS offsets).
#pragma unroll
  for (int s = 0; s < 16; ++s) asm volatile("" : "+v"(qb[s]));

  float m_ref = -INFINITY, l_run = 0.f;  // reference maximum (log2 units) and row sum
  f32x16 acc[kDim / 32];
#pragma unroll
  for (int d = 0; d < kDim / 32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;

  // the tokens this wave's rows hold (rows past ntok compute but are not stored)
  const int wave_first_tok = tok0 + wave * (kPRowsWave / kHeadsPerGroup);
  const int wave_last_tok = wave_first_tok + kPRowsWave / kHeadsPerGroup - 1;
  const bool wave_live = fits && wave * (kPRowsWave / kHeadsPerGroup) < ntok;
  // window rows see ring slots whose age (p0 - slot) mod 1024 is at most age_max;
  // wave_age_max is the smallest of those over the wave's rows
  const int age_max = min(p0, kWindow - 2 - my_tok);
  const int wave_age_max = min(p0, kWindow - 2 - wave_last_tok);

  // LDS operand offsets (bytes).  K (A of S^T = K Q^T): key rl, chunk 2s + hh, at
  // k_base + 32 s.
  // V^T (A of O^T = V^T P^T) by transposed reads: lane i of 16-lane group G points
  // at key 16j + 8r + 4(G/2) + i/4, dims 32d + 16(G%2) + 4(i%4) .. +3; the read
  // hands lane i dim 32d + 16(G%2) + i of the four keys 16j + 8r + 4(G/2) + 0..3.
  int k_base = (rl & 15) * kKPairBytes + (rl >> 4) * (2 * kDim) + 16 * hh;
  const int vg = lane >> 4, vi = lane & 15;
  const int v_key = 4 * (vg >> 1) + (vi >> 2);  // + 16j + 8r (keeps key & 3)
  const int v_dim = 16 * (vg & 1) + 4 * (vi & 3);  // + 32d
  // chunk 4d + x (x = v_dim / 8) sits at 4 (d ^ q) + x with q = key & 3, i.e. at the
  // lane's base for d % 4 plus 16 chunks (128 elements) per d / 4
  int v_addr[4];  // bytes
#pragma unroll
  for (int c = 0; c < 4; ++c)
    v_addr[c] = 2 * (v_key * kDim + ((4 * (c ^ (v_key & 3)) + (v_dim >> 3)) << 3) + (v_dim & 7));
  pf_vrd_tab[threadIdx.x] = pf_i32x4{v_addr[0], v_addr[1], v_addr[2], v_addr[3]};

  // One key tile on this wave's 32 rows: S^T = K Q^T (one MFMA chain over the 16
  // dim steps), mask, online softmax against a reference maximum that moves only
  // when a row's maximum grows by more than kPTau, O^T += V^T P^T.  The K offsets
  // pass through an opaque move per tile and the V^T offsets come from an LDS
  // table: hoisted out of the loop, each stage's base would occupy registers of
  // its own instead of folding into the LDS instructions' offsets.
#define PREFILL_COMPUTE_TILE(t, kt, vt)                                                      \
  {                                                                                          \
    PREFILL_TILE_SEG(t, csg, k0)                                                             \
    const int kind = csg.kind;                                                               \
    const int n = csg.n;                                                                     \
    if (wave_live && !(kind == 2 && k0 > wave_last_tok)) {                                   \
      asm volatile("" : "+v"(k_base));                                                       \
      f32x16 sc = {};                                                                        \
      _Pragma("unroll") for (int s = 0; s < 16; ++s) {                                       \
        const u32x4 kv = *reinterpret_cast<const u32x4 *>(                                   \
            reinterpret_cast<const char *>(kt) + k_base + 32 * s);                           \
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pbitcast<bf16x8>(kv), qb[s], sc, 0, 0,  \
                                                     0);                                     \
      }                                                                                      \
      /* key of register r: kl + 8(r/4) + r%4 */                                             \
      const int kl = k0 + 4 * hh;                                                            \
      if (kind == 1) {                                                                       \
        const int A = (p0 - k0) & (kWindow - 1);                                             \
        if (A < kPKeys - 1 || A > wave_age_max) {                                            \
          const int age0 = p0 - kl;                                                          \
          _Pragma("unroll") for (int r = 0; r < 16; ++r) {                                   \
            const int age = (age0 - (8 * (r >> 2) + (r & 3))) & (kWindow - 1);              \
            sc[r] = age <= age_max ? sc[r] : -INFINITY;                                      \
          }                                                                                  \
        }                                                                                    \
      } else if (kind == 2 ? k0 + kPKeys - 1 > wave_first_tok : k0 + kPKeys > n) {           \
        /* keys at or past lim are masked: the segment's end, or, in the chunk, the      */ \
        /* row's own token + 1 (the lane index from mbcnt: nothing kept live across the  */ \
        /* loop)                                                                         */ \
        const int ln_ = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));   \
        const int lim = kind == 2 ? wave_first_tok + ((ln_ & 31) >> 2) + 1 : n;              \
        _Pragma("unroll") for (int r = 0; r < 16; ++r) sc[r] =                               \
            kl + 8 * (r >> 2) + (r & 3) < lim ? sc[r] : -INFINITY;                           \
      }                                                                                      \
      float m8[8];                                                                           \
      _Pragma("unroll") for (int r = 0; r < 8; ++r) m8[r] = fmaxf(sc[r], sc[r + 8]);          \
      _Pragma("unroll") for (int r = 0; r < 4; ++r) m8[r] = fmaxf(m8[r], m8[r + 4]);          \
      float mt = fmaxf(fmaxf(m8[0], m8[2]), fmaxf(m8[1], m8[3]));                            \
      {                                                                                      \
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt),                 \
                                                         __float_as_uint(mt), false, false); \
        mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));                          \
      }                                                                                      \
      const bool move = mt > m_ref + kPTau;                                                  \
      const float m_use = move ? mt : m_ref;                                                 \
      const float alpha =                                                                    \
          (move && m_ref != -INFINITY) ? __builtin_amdgcn_exp2f(m_ref - m_use) : 1.f;        \
      if (__any(alpha != 1.f)) {                                                             \
        _Pragma("unroll") for (int d = 0; d < kDim / 32; ++d)                                \
            _Pragma("unroll") for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;               \
        l_run *= alpha;                                                                      \
      }                                                                                      \
      m_ref = m_use;                                                                         \
      const float m_sub = m_use == -INFINITY ? 0.f : m_use;                                  \
      u32x4 pw[2];                                                                           \
      _Pragma("unroll") for (int r = 0; r < 16; r += 2) pw[r >> 3][(r & 7) >> 1] =           \
          pack_bf16x2_hw(__builtin_amdgcn_exp2f(sc[r] - m_sub),                              \
                         __builtin_amdgcn_exp2f(sc[r + 1] - m_sub));                         \
      const pf_i32x4 vt4 = ((lds_vi32x4 *)pf_vrd_tab)[threadIdx.x];                            \
      const int va[4] = {vt4.x, vt4.y, vt4.z, vt4.w};                                        \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                        \
        const bf16x8 pb = pbitcast<bf16x8>(pw[j]);                                           \
        _Pragma("unroll") for (int d = 0; d < kDim / 32; ++d) {                              \
          const int vb = va[d & 3] + 2 * (128 * (d >> 2) + 16 * kDim * j);                   \
          const char *vp = reinterpret_cast<const char *>(vt) + vb;                          \
          const s16x4_t lohi[2] = {                                                          \
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vp)),                    \
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vp + 16 * kDim))};       \
          acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pbitcast<bf16x8>(lohi), pb,       \
                                                           acc[d], 0, 0, 0);                 \
        }                                                                                    \
      }                                                                                      \
      _Pragma("unroll") for (int q = 0; q < 8; ++q) l_run =                                  \
          __builtin_amdgcn_fdot2_f32_bf16(pbitcast<bf16x2_t>(pw[q >> 2][q & 3]), kOnesBf16x2, \
                                          l_run, false);                                     \
    }                                                                                        \
  }

  // One key tile: wait for its loads (this wave's, then everyone's via the
  // barrier), start the tile three ahead into the stage tile t - 1 used, compute.
#define PREFILL_STEP(t_, kt, vt, knext, vnext)                                               \
  if ((t_) < total) {                                                                        \
    const int t = (t_);                                                                      \
    /* this wave's loads of tile t are done once at most the later tiles' remain */          \
    const int later = min(total - 1 - t, kStages - 2);                                       \
    if (later >= 2)                                                                          \
      wait_vm_barrier<2 * kDmaPerTile>();                                                    \
    else if (later == 1)                                                                     \
      wait_vm_barrier<kDmaPerTile>();                                                        \
    else                                                                                     \
      wait_vm_barrier<0>();                                                                  \
    if (t + kStages - 1 < total) PREFILL_ISSUE_TILE(t + kStages - 1, knext, vnext);          \
    PREFILL_COMPUTE_TILE(t, kt, vt)                                                          \
  }

  for (int t0 = 0; t0 < total; t0 += kStages) {
    PREFILL_STEP(t0, pf_k0, pf_v0, pf_k3, pf_v3)
    PREFILL_STEP(t0 + 1, pf_k1, pf_v1, pf_k0, pf_v0)
    PREFILL_STEP(t0 + 2, pf_k2, pf_v2, pf_k1, pf_v1)
    PREFILL_STEP(t0 + 3, pf_k3, pf_v3, pf_k2, pf_v2)
  }
#undef PREFILL_STEP
#undef PREFILL_COMPUTE_TILE
#undef PREFILL_TILE_SEG
#undef PREFILL_ISSUE_TILE

  // epilogue: row rl = token my_tok, head my_head; lanes rl and rl + 32 hold the
  // two halves of each 8-dim run
  float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (my_tl < ntok) {
    const int head = g * kHeadsPerGroup + my_head;
    uint16_t *o = (anchor ? a.o_rma : a.o_win) +
                  ((static_cast<size_t>(b) * a.chunk + my_tok) * kHeads + head) * kDim;
    const bool empty = m_ref == -INFINITY;
    const float inv = empty ? 0.f : 1.f / l_tot;
#pragma unroll
    for (int d = 0; d < kDim / 32; ++d) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2 ov = make_uint2(0u, 0u);
        if (!empty) {
          ov.x = pack_bf16x2_hw(acc[d][4 * q] * inv, acc[d][4 * q + 1] * inv);
          ov.y = pack_bf16x2_hw(acc[d][4 * q + 2] * inv, acc[d][4 * q + 3] * inv);
        }
        *reinterpret_cast<uint2 *>(o + 32 * d + 8 * q + 4 * hh) = ov;
      }
    }
    if (hh == 0) {
      float *lse = (anchor ? a.lse_rma : a.lse_win) +
                   (static_cast<size_t>(b) * a.chunk + my_tok) * kHeads + head;
      *lse = empty ? -INFINITY : (m_ref + log2f(l_tot)) * kPLn2;
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
