// Decode-step attention of one SWA||RMA layer on gfx950.
//
// What it computes (fluxbbs.com "EdgeRock-4B 开源：72 MiB 固定 KV，AIME 82.9 分",
// section "架构：递归、局部窗口与记忆锚点三件套"): 16 query heads over 4 KV groups
// of width 256 read two branches in parallel -- the 1024-slot sliding window and
// the anchor records (committed bank, then the pending block) -- with learned RMS
// norm on the query, rotary on dims 0..63 (base 1e7) and softmax scale 1/16.
// Each branch returns its output and natural-log log-sum-exp.
//
// Design.  The step reads 9 MiB of BF16 K/V per (sequence, layer) against
// 4 flop/byte, so it is bound by HBM bandwidth; the kernel is built to stream
// every K/V byte exactly once:
//  * one workgroup (4 waves) per (branch, sequence, KV group, key-range split);
//    the 4 query heads of a group share every K/V row they read.
//  * each wave walks 16-key tiles; K rows go straight from HBM into the A
//    operand of v_mfma_f32_16x16x32_bf16 (each lane loads 16 contiguous bytes;
//    the head dim is the contraction, so no reshuffle is needed), giving the
//    scores of 16 keys x 4 heads in one 4-register accumulator.
//  * V rows are loaded with coalesced 16-byte loads, staged in the wave's own
//    LDS rows and read back with transposed 8-byte LDS reads as the A operand of
//    v_mfma_f32_16x16x16bf16_1k (contraction over keys); P (BF16) is the B
//    operand and comes straight from the score accumulator's registers.
//  * online softmax per head in the log2 domain: the scaled query carries
//    log2(e)/16, so probabilities are exp2(s - m).
//  * K and V reach registers through buffer loads whose range is the valid rows
//    of the segment, so rows past the end read as zero; as soon as a tile's K
//    and V are consumed (V copied to LDS, scores formed) the next tile's loads
//    are issued, and they fly while the softmax update and P x V run.
//  * waves merge through LDS; with several splits a second kernel merges the
//    splits' (m, l, acc) partials.
//
// FP8 variant (rows of 256 E4M3 codes plus one FP32 scale): 32-key tiles keep
// the same bytes in flight per wave; codes are widened to BF16 exactly with the
// hardware conversion and fed to the same MFMAs: K codes as they arrive, V codes
// after an 8-bit transposing LDS read (V stays E4M3 in LDS, half the bytes of a
// widened tile), the 32 keys forming one 32-long contraction for P x V; the K scale
// multiplies each score and the V scale each probability weight.
#include <atomic>
#include <mutex>

#include "rma_device.h"

namespace rma {

// Two floats -> packed BF16 pair with the hardware conversion (v_cvt_pk_bf16_f32,
// round to nearest even): the same bits as pack_bf16x2 for every input but NaN, in
// one instruction instead of about ten.
__device__ __forceinline__ uint32_t pack_bf16x2_cvt(float lo, float hi) {
  typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
  const bf16x2_cvt_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

constexpr int kTile = 16;
#ifndef RMA_DECODE_WAVES
#define RMA_DECODE_WAVES 4
#endif
constexpr int kWaves = RMA_DECODE_WAVES;  // waves per workgroup, all on one (branch, seq, group)
constexpr int kThreads = 64 * kWaves;
constexpr int kMergeThreads = 64 * kHeadsPerGroup;
static_assert(kWaves >= kHeadsPerGroup, "one wave per head in the query prologue and epilogue");
// LDS row stride of a staged V tile, in elements: 544 bytes, so rows start 8 banks
// apart and a transposed read of 8 rows x 32 bytes hits 64 distinct banks.
constexpr int kVStride = kDim + 16;
constexpr int kPartStride = 4 + kDim;
constexpr int kMaxSplits = 16;  // batch 1: 8 units x 16 = 128 workgroups, 16 per XCD
#ifndef RMA_DECODE_MIN_WGS
#define RMA_DECODE_MIN_WGS 512
#endif
// Split each branch only until a launch has two workgroups per CU (256 CUs):
// more, smaller workgroups measured slower at batch 64 and 512 (per-workgroup
// prologue, partial writes and the merge launch cost more than they balance).
constexpr int kMinWorkgroups = RMA_DECODE_MIN_WGS;
constexpr float kQScale = 1.4426950408889634f / 16.0f;  // log2(e) / sqrt(256)
constexpr float kLn2 = 0.69314718055994531f;
// Row offset of a load that must go out without touching memory (past every
// segment, so the range check returns zeros): a load issued on every path keeps the
// compiler's wait counts exact.
constexpr int kNoRows = 1 << 20;
// Cache policy of the K/V loads: non-temporal (every byte is read exactly once per
// step, so it should not displace anything in the caches).
constexpr int kStream = 2;

// K/V rows are BF16 (512 bytes) or, in the FP8 variant, E4M3 codes (256 bytes) with
// one FP32 scale per row in the *_ks / *_vs arrays.
struct DecodeParams {
  const uint8_t *win_k, *win_v, *bank_k, *bank_v, *pend_k, *pend_v;
  const float *win_ks, *win_vs, *bank_ks, *bank_vs, *pend_ks, *pend_vs;
  const int32_t *n_bank, *n_pend, *pos;
  const uint16_t *q_win, *q_rma;
  const float *gq_win, *gq_rma;
  float eps;
  double rope_ratio;  // base^(-1/32)
  uint16_t *o_win, *o_rma;
  float *lse_win, *lse_rma;
  float *part;
  int batch, splits;
};

// One contiguous run of valid key rows (the window, the bank, or the pending
// block of one sequence and group), addressed through buffer resources whose
// size is the valid byte count.  The hardware checks the range per dword with the
// scalar offset included, so rows (and scales) past the end read as zero.
struct Segment {
  __amdgpu_buffer_rsrc_t k, v;
  __amdgpu_buffer_rsrc_t ks, vs;  // FP8 variant: per-row scales
  int n;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

template <typename T, typename F>
__device__ __forceinline__ T bitcast(const F &f) {
  return __builtin_bit_cast(T, f);
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// The staged query block: rows 0..3 hold the group's four scaled queries, rows
// 4..15 stay zero (the score MFMA is 16 wide).  Rows are padded to 528 bytes so
// that the 16 lanes reading one 16-byte column from 16 rows hit 16 distinct
// groups of four banks.
constexpr int kQStride = kDim + 8;

struct SoftmaxState {
  float m, l;
  f32x4 acc[16];
};

// ---------------------------------------------------------------- setup and epilogue
// Workgroup -> (unit, split).  Workgroups are handed to the 8 XCDs in turn, so the
// splits of one unit are numbered 8 apart: they all run on one XCD, whose L2 then
// still holds their partials when the merge workgroup of that unit (number = unit,
// the same XCD) reads them.  Units come in multiples of 8 (2 branches x 4 groups per
// sequence), so the map is a bijection; without splits it is the identity.
constexpr int kXcds = 8;
static_assert(2 * kGroups % kXcds == 0, "units per sequence are a multiple of the XCD count");
__device__ __forceinline__ void unit_split_of(int wg, int splits, int &unit, int &split) {
  const int xcd = wg % kXcds, slot = wg / kXcds;
  unit = (slot / splits) * kXcds + xcd;
  split = slot % splits;
}
// The key segments of one (branch, sequence, group) for position p and the given
// bank and pending counts; rb = bytes per row.
template <bool kFp8>
__device__ __forceinline__ void unit_segments_at(const DecodeParams &a, int b, int g, bool anchor,
                                                 int p, int n_bank, int n_pend, Segment &seg0,
                                                 Segment &seg1) {
  constexpr int rb = kFp8 ? kDim : 2 * kDim;
  const size_t sgi = static_cast<size_t>(b) * kGroups + g;
  if (anchor) {
    // uniform values, kept scalar so that the buffer resources stay in scalar registers
    const int nb = __builtin_amdgcn_readfirstlane(min(max(n_bank, 0), kBank));
    const int np = __builtin_amdgcn_readfirstlane(min(max(n_pend, 0), kBlock));
    seg0.k = make_rsrc(a.bank_k + sgi * kBank * rb, nb * rb);
    seg0.v = make_rsrc(a.bank_v + sgi * kBank * rb, nb * rb);
    seg0.n = nb;
    seg1.k = make_rsrc(a.pend_k + sgi * kBlock * rb, np * rb);
    seg1.v = make_rsrc(a.pend_v + sgi * kBlock * rb, np * rb);
    seg1.n = np;
    if constexpr (kFp8) {
      seg0.ks = make_rsrc(a.bank_ks + sgi * kBank, nb * 4);
      seg0.vs = make_rsrc(a.bank_vs + sgi * kBank, nb * 4);
      seg1.ks = make_rsrc(a.pend_ks + sgi * kBlock, np * 4);
      seg1.vs = make_rsrc(a.pend_vs + sgi * kBlock, np * 4);
    }
  } else {
    const int nw = __builtin_amdgcn_readfirstlane(min(max(p + 1, 0), kWindow));
    seg0.k = make_rsrc(a.win_k + sgi * kWindow * rb, nw * rb);
    seg0.v = make_rsrc(a.win_v + sgi * kWindow * rb, nw * rb);
    seg0.n = nw;
    if constexpr (kFp8) {
      seg0.ks = make_rsrc(a.win_ks + sgi * kWindow, nw * 4);
      seg0.vs = make_rsrc(a.win_vs + sgi * kWindow, nw * 4);
    }
    seg1 = seg0;
    seg1.n = 0;
  }
}

// The key segments as the state holds them.
template <bool kFp8>
__device__ __forceinline__ void unit_segments(const DecodeParams &a, int b, int g, bool anchor,
                                              Segment &seg0, Segment &seg1) {
  if (anchor)
    unit_segments_at<kFp8>(a, b, g, true, 0, a.n_bank[b], a.n_pend[b], seg0, seg1);
  else
    unit_segments_at<kFp8>(a, b, g, false, a.pos[b], 0, 0, seg0, seg1);
}

// The raw query elements of wave w (head 4g + w, dims 4*lane..4*lane+3) and the
// lane's four query gains.  Issued first in a kernel, their wait does not cover the
// key loads issued after them.
static_assert(kWaves == kHeadsPerGroup, "one wave per head of the group");
struct QueryRaw {
  uint2 q;
  float4 gain;
};

__device__ __forceinline__ QueryRaw load_query(const DecodeParams &a, int b, int g, bool anchor,
                                               int wave, int lane) {
  const uint16_t *q = (anchor ? a.q_rma : a.q_win) +
                      (static_cast<size_t>(b) * kHeads + g * kHeadsPerGroup + wave) * kDim;
  QueryRaw r;
  r.q = *reinterpret_cast<const uint2 *>(q + 4 * lane);
  r.gain = *reinterpret_cast<const float4 *>((anchor ? a.gq_rma : a.gq_win) + 4 * lane);
  return r;
}

// Query prep at position p from the raw elements: wave w normalises, rotates and
// scales head 4g + w into q_lds row w; the other rows are zeroed.  The gains go
// through the wave's own LDS row (g_row, kDim floats), so the norm reads them there
// rather than from memory.  Ends with a workgroup barrier.
__device__ __forceinline__ void stage_query_raw(const DecodeParams &a, const QueryRaw &raw,
                                                int p, int wave, int lane,
                                                uint16_t (*q_lds)[kQStride], float *g_row) {
  {
    *reinterpret_cast<float4 *>(g_row + 4 * lane) = raw.gain;
    float x[4] = {bf16_lo(raw.q.x), bf16_hi(raw.q.x), bf16_lo(raw.q.y), bf16_hi(raw.q.y)};
    float c, sn;
    rope_cos_sin(a.rope_ratio, p, lane, c, sn);
    norm_rope_head(x, g_row, a.eps, c, sn, lane);
    uint2 o;
    o.x = pack_bf16x2(x[0] * kQScale, x[1] * kQScale);
    o.y = pack_bf16x2(x[2] * kQScale, x[3] * kQScale);
    *reinterpret_cast<uint2 *>(&q_lds[wave][4 * lane]) = o;
  }
  for (int i = threadIdx.x; i < 12 * kQStride / 4; i += kThreads)
    reinterpret_cast<uint2 *>(&q_lds[kHeadsPerGroup][0])[i] = make_uint2(0, 0);
  __syncthreads();
}

__device__ __forceinline__ void stage_query(const DecodeParams &a, int b, int g, bool anchor,
                                            int p, int wave, int lane,
                                            uint16_t (*q_lds)[kQStride], float *g_row) {
  stage_query_raw(a, load_query(a, b, g, anchor, wave, lane), p, wave, lane, q_lds, g_row);
}

// Merge the four waves' partial softmax states through LDS (macc: 16 KiB that no
// wave reads any more) and write the output, or this split's partial.
__device__ __forceinline__ void finish_unit(const DecodeParams &a, const SoftmaxState &st,
                                            float *macc, float (*red_m)[kHeadsPerGroup],
                                            float (*red_l)[kHeadsPerGroup], int wave, int lane,
                                            int unit, int split, bool anchor, int b, int g) {
  // Sum the denominators of the four lanes that share a head.
  float l_tot = st.l + __shfl_xor(st.l, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  {
    const int hh = lane & 15, kg = lane >> 4;
    if (hh < kHeadsPerGroup) {
      float *dst = macc + (wave * kHeadsPerGroup + hh) * kDim + 4 * kg;
#pragma unroll
      for (int db = 0; db < 16; ++db)
        *reinterpret_cast<float4 *>(dst + 16 * db) =
            make_float4(st.acc[db][0], st.acc[db][1], st.acc[db][2], st.acc[db][3]);
      if (kg == 0) {
        red_m[wave][hh] = st.m;
        red_l[wave][hh] = l_tot;
      }
    }
  }
  __syncthreads();

  if (wave >= kHeadsPerGroup) return;
  const int h = wave;  // this wave now owns head 4g + h, dims 4*lane..4*lane+3
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][h]);
  float L = 0.f;
  float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = red_m[w][h];
      const float wt = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += red_l[w][h] * wt;
      const float4 v = *reinterpret_cast<const float4 *>(macc + (w * kHeadsPerGroup + h) * kDim +
                                                         4 * lane);
      O.x += v.x * wt;
      O.y += v.y * wt;
      O.z += v.z * wt;
      O.w += v.w * wt;
    }
  }
  const int head = g * kHeadsPerGroup + h;
  if (a.splits == 1) {
    uint16_t *o = (anchor ? a.o_rma : a.o_win) + (static_cast<size_t>(b) * kHeads + head) * kDim;
    float *lse = (anchor ? a.lse_rma : a.lse_win) + static_cast<size_t>(b) * kHeads + head;
    uint2 ov = make_uint2(0, 0);
    float lv = -INFINITY;
    if (M != -INFINITY) {
      const float inv = 1.f / L;
      ov.x = pack_bf16x2(O.x * inv, O.y * inv);
      ov.y = pack_bf16x2(O.z * inv, O.w * inv);
      lv = (M + log2f(L)) * kLn2;
    }
    *reinterpret_cast<uint2 *>(o + 4 * lane) = ov;
    if (lane == 0) *lse = lv;
  } else {
    float *pp = a.part + (static_cast<size_t>(unit * a.splits + split) * kHeadsPerGroup + h) *
                             kPartStride;
    if (lane == 0) {
      pp[0] = M;
      pp[1] = L;
    }
    *reinterpret_cast<float4 *>(pp + 4 + 4 * lane) = O;
  }
}

// ---------------------------------------------------------------- BF16 rows
// Issue the loads of one 16-key tile starting at row key0 of a segment: K as MFMA
// A operands (lane: row key0 + lane%16, dims 32s + 8(lane/16) .. +8), V as row
// chunks (lane: row key0 + 2i + lane/32, dims 8(lane%32) .. +8).
__device__ __forceinline__ void load_tile(const Segment &sg, int key0, int lane, uint4 (&K)[8],
                                          uint4 (&V)[8]) {
  const int hh = lane & 15, kg = lane >> 4;
  const int koff = hh * (kDim * 2) + kg * 16;
  const int voff = (lane >> 5) * (kDim * 2) + (lane & 31) * 16;
  const int soff = key0 * (kDim * 2);
#pragma unroll
  for (int s = 0; s < 8; ++s)
    K[s] = bitcast<uint4>(__builtin_amdgcn_raw_buffer_load_b128(sg.k, koff + 64 * s, soff, kStream));
#pragma unroll
  for (int i = 0; i < 8; ++i)
    V[i] = bitcast<uint4>(
        __builtin_amdgcn_raw_buffer_load_b128(sg.v, voff + 2 * kDim * 2 * i, soff, kStream));
}

// Stage V in LDS and form the scores of one tile (consumes K and V).
__device__ __forceinline__ f32x4 scores_tile(int nvalid, int lane, const uint4 (&K)[8],
                                             const uint4 (&V)[8], const bf16x8 (&qv)[8],
                                             uint16_t *vl) {
  const int kg = lane >> 4;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint4 *>(vl + (2 * i + (lane >> 5)) * kVStride + 8 * (lane & 31)) = V[i];
  // D[key][head] = sum_d K[key][d] * qhat[head][d]; the B operand is the staged
  // query block (head hh; rows >= 4 are zero).  Lane holds keys 4kg..4kg+3 of head hh.
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 8; ++s)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(K[s]), qv[s], sc, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (4 * kg + i >= nvalid) sc[i] = -INFINITY;
  return sc;
}

// Online-softmax update and P x V for one tile whose V rows are staged in LDS.
__device__ __forceinline__ void accumulate_tile(f32x4 sc, int lane, const uint16_t *vl,
                                                SoftmaxState &st) {
  const int kg = lane >> 4;
  float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float m_new = fmaxf(st.m, mt);
  float alpha = 1.f;
  uint32_t pw0 = 0, pw1 = 0;
  float psum = 0.f;
  if (m_new != -INFINITY) {
    alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    pw0 = pack_bf16x2_cvt(__builtin_amdgcn_exp2f(sc[0] - m_new),
                          __builtin_amdgcn_exp2f(sc[1] - m_new));
    pw1 = pack_bf16x2_cvt(__builtin_amdgcn_exp2f(sc[2] - m_new),
                          __builtin_amdgcn_exp2f(sc[3] - m_new));
    // the denominator uses the same rounded weights as the numerator
    psum = (bf16_lo(pw0) + bf16_hi(pw0)) + (bf16_lo(pw1) + bf16_hi(pw1));
  }
  // rescale the accumulators only when some head's running maximum moved (alpha
  // is exactly 1 otherwise)
  if (__any(m_new != st.m)) {
#pragma unroll
    for (int db = 0; db < 16; ++db) st.acc[db] *= alpha;
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
  const s16x4 pb = bitcast<s16x4>(make_uint2(pw0, pw1));
  // D[dim][head] += sum_key V[key][dim] * P[head][key].  This wave's LDS reads
  // follow its own writes in scores_tile (LDS runs a wave's operations in order).
  // Transposed read: lane r of group kg supplies row 4kg + r/4, dims 4(r%4) .. +4 of
  // a 16-dim block and receives dim r of rows 4kg .. 4kg+3.
  const int r = lane & 15;
  const uint16_t *src = vl + (4 * kg + (r >> 2)) * kVStride + 4 * (r & 3);
#pragma unroll
  for (int db = 0; db < 16; ++db) {
    const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + 16 * db));
    st.acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, st.acc[db], 0, 0, 0);
  }
}

__global__ __launch_bounds__(kThreads, 2) void decode_attn_kernel(DecodeParams a) {
  __shared__ __align__(16) uint16_t v_lds[kWaves][kTile * kVStride];
  __shared__ __align__(16) uint16_t q_lds[16][kQStride];  // rows 4..15 stay zero
  __shared__ __align__(16) float g_lds[kWaves][kDim];
  __shared__ float red_m[kWaves][kHeadsPerGroup], red_l[kWaves][kHeadsPerGroup];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps tile selection scalar
  int unit, split;
  unit_split_of(blockIdx.x, a.splits, unit, split);
  const int per_branch = a.batch * kGroups;
  const bool anchor = unit < per_branch;  // anchor units first: they are the longer ones
  const int bg = anchor ? unit : unit - per_branch;
  const int b = bg / kGroups, g = bg % kGroups;

  Segment seg0, seg1;
  unit_segments<false>(a, b, g, anchor, seg0, seg1);
  // Tiles of segment 0 come first, then those of segment 1; each tile lies in one
  // segment.  This workgroup takes tiles [tb, te).
  const int T0 = (seg0.n + kTile - 1) / kTile;
  const int T = T0 + (seg1.n + kTile - 1) / kTile;
  const int per = (T + a.splits - 1) / a.splits;
  const int tb = split * per;
  const int te = min(T, tb + per);

  SoftmaxState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int d = 0; d < 16; ++d) st.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint16_t *vl = v_lds[wave];
  uint4 K[8], V[8];
  int t = tb + wave;
  // The query's loads go first and the first tile's right after them (on every
  // path): the prologue waits for the query alone, and its norm and rotary work
  // overlaps the tile's loads.
  const QueryRaw qraw = load_query(a, b, g, anchor, wave, lane);
  load_tile(t < T0 ? seg0 : seg1, t < te ? (t < T0 ? t : t - T0) * kTile : kNoRows, lane, K, V);
  stage_query_raw(a, qraw, a.pos[b], wave, lane, q_lds, g_lds[wave]);
  // The query operands stay in registers for the whole key loop: lane (hh, kg) holds
  // dims 32s + 8kg .. +8 of head hh (rows >= 4 are zero).
  bf16x8 qv[8];
  {
    const uint16_t *qrow = &q_lds[0][0] + (lane & 15) * kQStride + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 8; ++s) qv[s] = bitcast<bf16x8>(*reinterpret_cast<const uint4 *>(qrow + 32 * s));
  }

  for (; t < te; t += kWaves) {
    const int key0 = (t < T0 ? t : t - T0) * kTile;
    const int nvalid = (t < T0 ? seg0.n : seg1.n) - key0;
    const f32x4 sc = scores_tile(nvalid, lane, K, V, qv, vl);
    // K and V are consumed: the next tile's loads fly while this one accumulates.
    const int tn = t + kWaves;
    if (tn < te) load_tile(tn < T0 ? seg0 : seg1, (tn < T0 ? tn : tn - T0) * kTile, lane, K, V);
    accumulate_tile(sc, lane, vl, st);
  }

  __syncthreads();  // every wave is done with its V rows; reuse them for the merge
  finish_unit(a, st, reinterpret_cast<float *>(&v_lds[0][0]), red_m, red_l, wave, lane, unit,
              split, anchor, b, g);
}

// ---------------------------------------------------------------- fused step
// One token per sequence, appended and attended in one launch: the same result as
// swa_rma_append followed by swa_rma_decode_attn (fluxbbs.com page, section
// "架构：递归、局部窗口与记忆锚点三件套": keys normed and rotated at their own
// position, values raw; neodrop.ai repost, section "三段记忆，只记值得记的": one
// candidate per token into the pending block).
//  * every workgroup reads pos and n_pend as they were and counts the new token in
//    its segments (window slot p mod 1024, pending row n_pend);
//  * the workgroup whose tiles hold a branch's new row forms that row (norm +
//    rotary of the key, the value as given), writes it to the state and puts it in
//    its tile registers in place of what the loads read from that row;
//  * the last workgroup of a sequence to finish (a counter per sequence in the
//    workspace) advances pos and n_pend and records the source position and
//    score, after every workgroup of the sequence has read them.  No data passes
//    between workgroups of the launch, so no cross-workgroup fence is needed.
struct StepParams {
  DecodeParams d;
  uint16_t *win_k, *win_v, *pend_k, *pend_v;
  float *pend_score;
  int32_t *pend_src, *n_pend, *pos;
  const uint16_t *k_win, *v_win, *k_rma, *v_rma;  // [B][4][256], raw
  const float *score;                             // [B][4] or null
  const float *gk_win, *gk_rma;
  uint32_t *done;                                 // [B], zero between launches
};

__global__ __launch_bounds__(kThreads, 2) void decode_step_kernel(StepParams sp) {
  const DecodeParams &a = sp.d;
  __shared__ __align__(16) uint16_t v_lds[kWaves][kTile * kVStride];
  __shared__ __align__(16) uint16_t q_lds[16][kQStride];
  __shared__ __align__(16) uint16_t patch[2][kDim];  // the new K and V rows
  __shared__ __align__(16) float g_lds[kWaves + 1][kDim];  // query gains per wave, key gains
  __shared__ float red_m[kWaves][kHeadsPerGroup], red_l[kWaves][kHeadsPerGroup];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int unit, split;
  unit_split_of(blockIdx.x, a.splits, unit, split);
  const int per_branch = a.batch * kGroups;
  const bool anchor = unit < per_branch;
  const int bg = anchor ? unit : unit - per_branch;
  const int b = bg / kGroups, g = bg % kGroups;

  // The query and the token's records do not depend on the state: their loads go
  // first, so that waiting for them does not wait for the key loads, and the norm
  // and rotary work overlaps those loads.
  const QueryRaw qraw = load_query(a, b, g, anchor, wave, lane);
  const size_t rec_in = (static_cast<size_t>(b) * kGroups + g) * kDim + 4 * lane;
  const uint2 krec_raw = *reinterpret_cast<const uint2 *>((anchor ? sp.k_rma : sp.k_win) + rec_in);
  const uint2 vrec_raw = *reinterpret_cast<const uint2 *>((anchor ? sp.v_rma : sp.v_win) + rec_in);
  const float4 kgain = *reinterpret_cast<const float4 *>((anchor ? sp.gk_rma : sp.gk_win) + 4 * lane);

  // the state before the token; a full pending block takes no token (as in append)
  const int p_old = a.pos[b];
  const int np_old = a.n_pend[b];
  const bool app = np_old >= 0 && np_old < kBlock;
  const int p = app ? p_old + 1 : p_old;
  const int nb = anchor ? min(max(a.n_bank[b], 0), kBank) : 0;

  Segment seg0, seg1;
  unit_segments_at<false>(a, b, g, anchor, p, nb, app ? np_old + 1 : np_old, seg0, seg1);
  const int T0 = (seg0.n + kTile - 1) / kTile;
  const int T = T0 + (seg1.n + kTile - 1) / kTile;
  const int per = (T + a.splits - 1) / a.splits;
  const int tb = split * per;
  const int te = min(T, tb + per);
  // the tile and row of this branch's new key
  const int new_key = anchor ? np_old : (p & (kWindow - 1));
  const int new_tile = app ? (anchor ? T0 : 0) + new_key / kTile : -1;
  const int new_off = new_key % kTile;
  const bool owner = new_tile >= tb && new_tile < te;

  SoftmaxState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int d = 0; d < 16; ++d) st.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint16_t *vl = v_lds[wave];
  uint4 K[8], V[8];
  int t = tb + wave;
  load_tile(t < T0 ? seg0 : seg1, t < te ? (t < T0 ? t : t - T0) * kTile : kNoRows, lane, K, V);
  // the owner's wave 0 forms the new rows; stage_query's barrier publishes the patch
  if (owner && wave == 0) {
    const uint2 kr = krec_raw;
    const uint2 vr = vrec_raw;
    float x[4] = {bf16_lo(kr.x), bf16_hi(kr.x), bf16_lo(kr.y), bf16_hi(kr.y)};
    float c, sn;
    rope_cos_sin(a.rope_ratio, p, lane, c, sn);
    *reinterpret_cast<float4 *>(&g_lds[kWaves][4 * lane]) = kgain;
    norm_rope_head(x, &g_lds[kWaves][0], a.eps, c, sn, lane);
    const uint2 kw = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
    *reinterpret_cast<uint2 *>(&patch[0][4 * lane]) = kw;
    *reinterpret_cast<uint2 *>(&patch[1][4 * lane]) = vr;
    const size_t sgi = static_cast<size_t>(b) * kGroups + g;
    const size_t row = anchor ? (sgi * kBlock + np_old) * kDim : (sgi * kWindow + new_key) * kDim;
    *reinterpret_cast<uint2 *>((anchor ? sp.pend_k : sp.win_k) + row + 4 * lane) = kw;
    *reinterpret_cast<uint2 *>((anchor ? sp.pend_v : sp.win_v) + row + 4 * lane) = vr;
  }
  stage_query_raw(a, qraw, p, wave, lane, q_lds, g_lds[wave]);
  bf16x8 qv[8];
  {
    const uint16_t *qrow = &q_lds[0][0] + (lane & 15) * kQStride + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 8; ++s) qv[s] = bitcast<bf16x8>(*reinterpret_cast<const uint4 *>(qrow + 32 * s));
  }

  for (; t < te; t += kWaves) {
    const int key0 = (t < T0 ? t : t - T0) * kTile;
    const int nvalid = (t < T0 ? seg0.n : seg1.n) - key0;
    if (t == new_tile) {
      // the new row replaces whatever the loads read from it (lane: key lane % 16
      // for K, rows 2i + lane / 32 for V)
      if ((lane & 15) == new_off) {
#pragma unroll
        for (int s = 0; s < 8; ++s)
          K[s] = *reinterpret_cast<const uint4 *>(&patch[0][32 * s + 8 * (lane >> 4)]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (2 * i + (lane >> 5) == new_off)
          V[i] = *reinterpret_cast<const uint4 *>(&patch[1][8 * (lane & 31)]);
    }
    const f32x4 sc = scores_tile(nvalid, lane, K, V, qv, vl);
    const int tn = t + kWaves;
    if (tn < te) load_tile(tn < T0 ? seg0 : seg1, (tn < T0 ? tn : tn - T0) * kTile, lane, K, V);
    accumulate_tile(sc, lane, vl, st);
  }

  __syncthreads();
  finish_unit(a, st, reinterpret_cast<float *>(&v_lds[0][0]), red_m, red_l, wave, lane, unit,
              split, anchor, b, g);
  // every workgroup of the sequence has read pos / n_pend once its count is in
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t nwg = 2u * kGroups * static_cast<uint32_t>(a.splits);
    if (atomicAdd(&sp.done[b], 1u) == nwg - 1) {
      sp.done[b] = 0u;
      if (app) {
        sp.pend_src[static_cast<size_t>(b) * kBlock + np_old] = p;
        if (sp.score) {
#pragma unroll
          for (int gg = 0; gg < kGroups; ++gg)
            sp.pend_score[(static_cast<size_t>(b) * kBlock + np_old) * kGroups + gg] =
                sp.score[b * kGroups + gg];
        }
        sp.n_pend[b] = np_old + 1;
        sp.pos[b] = p;
      }
    }
  }
}

// ---------------------------------------------------------------- FP8 rows
// A tile holds 32 keys, so a wave keeps 16 KiB of codes in flight, as a BF16 tile
// of 16 keys does: half the bytes per key would otherwise halve the bytes in
// flight, and with them the bandwidth a latency-bound stream reaches.  Codes are
// widened to BF16 (exactly) for the same MFMAs; the K scale multiplies the score
// and the V scale the probability weight of its key.
constexpr int kTile8 = 32;

// Eight E4M3 codes (two words) -> eight BF16 values.
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  return make_uint4(bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                    bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                    bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                    bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true)));
}

// Eight signed 8-bit codes (two words, byte i = code i) -> eight BF16 values: each
// code converts exactly (|code| <= 127 has at most 7 significant bits).
__device__ __forceinline__ uint4 i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = static_cast<float>(static_cast<int8_t>(lo >> (8 * i)));
    f[4 + i] = static_cast<float>(static_cast<int8_t>(hi >> (8 * i)));
  }
  return make_uint4(pack_bf16x2_cvt(f[0], f[1]), pack_bf16x2_cvt(f[2], f[3]),
                    pack_bf16x2_cvt(f[4], f[5]), pack_bf16x2_cvt(f[6], f[7]));
}

// The widening of the 8-bit variant in use: E4M3 codes or INT8 codes.
template <bool kInt8>
__device__ __forceinline__ uint4 q8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  if constexpr (kInt8)
    return i8x8_to_bf16x8(lo, hi);
  else
    return e4m3x8_to_bf16x8(lo, hi);
}

// Loads of one 32-key tile at row key0 of a segment (16-byte loads throughout):
//  K[4u + s]: key key0 + 16u + lane%16, codes of dims 64s + 16(lane/16) .. +16;
//  V[i]:      row key0 + 4i + lane/16, codes of dims 16(lane%16) .. +16;
//  ks[u], vs[u]: scales of keys key0 + 16u + 4(lane/16) .. +4 (the lane's score keys).
// The K and V halves are issued separately: each half's next loads go out as soon
// as its registers are consumed.
__device__ __forceinline__ void load_k_fp8(const Segment &sg, int key0, int lane, uint4 (&K)[8]) {
  const int hh = lane & 15, kg = lane >> 4;
  const int soff = key0 * kDim;
  const int koff = hh * kDim + 16 * kg;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      K[4 * u + s] = bitcast<uint4>(__builtin_amdgcn_raw_buffer_load_b128(
          sg.k, koff + 16 * u * kDim + 64 * s, soff, kStream));
}

__device__ __forceinline__ void load_v_fp8(const Segment &sg, int key0, int lane, uint4 (&V)[8]) {
  const int soff = key0 * kDim;
  const int voff = (lane >> 4) * kDim + 16 * (lane & 15);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    V[i] = bitcast<uint4>(
        __builtin_amdgcn_raw_buffer_load_b128(sg.v, voff + 4 * i * kDim, soff, kStream));
}

// The K and V scales of a workgroup's tiles [tb, te) go to LDS once, before the key
// loop, as two contiguous runs read by the whole workgroup (16 bytes a thread):
// per-tile loads of 128 bytes each from the two scale arrays cost more than their
// share of the bytes.  Entry 32(t - tb) + i holds key i of tile t; keys past a
// segment's end read as zero.
constexpr int kMaxScaleKeys = (kBank + kBlock) / kTile8 * kTile8;  // a whole anchor unit
__device__ __forceinline__ void load_scale_run(const Segment &sg, int row0, int n4, float *ks_l,
                                               float *vs_l) {
  for (int i = threadIdx.x; i < n4; i += kThreads) {
    const f32x4 k4 = bitcast<f32x4>(__builtin_amdgcn_raw_buffer_load_b128(sg.ks, 16 * i, row0 * 4, kStream));
    const f32x4 v4 = bitcast<f32x4>(__builtin_amdgcn_raw_buffer_load_b128(sg.vs, 16 * i, row0 * 4, kStream));
    *reinterpret_cast<f32x4 *>(ks_l + 4 * i) = k4;
    *reinterpret_cast<f32x4 *>(vs_l + 4 * i) = v4;
  }
}

__device__ __forceinline__ void load_scales_fp8(const Segment &seg0, const Segment &seg1, int T0,
                                                int tb, int te, float *ks_l, float *vs_l) {
  // tiles [tb, min(te, T0)) of segment 0, then [max(tb, T0), te) of segment 1
  const int e0 = min(te, T0), b1 = max(tb, T0);
  if (tb < e0) load_scale_run(seg0, tb * kTile8, (e0 - tb) * (kTile8 / 4), ks_l, vs_l);
  if (b1 < te)
    load_scale_run(seg1, (b1 - T0) * kTile8, (te - b1) * (kTile8 / 4), ks_l + (b1 - tb) * kTile8,
                   vs_l + (b1 - tb) * kTile8);
}

// The same runs through registers: this thread's 16-byte piece of each run (a run
// is at most 1024 keys, 256 pieces), loaded after the first tile's loads and stored
// after the query prologue.  The INT8 decode, with more vector work per tile, gains
// from not waiting for the scales before its first tile goes out; the E4M3 decode
// does not (measured both ways).
struct ScalePieces {
  f32x4 k0, v0, k1, v1;
  int i0, i1;  // LDS float index of each piece, -1 if none
};
static_assert(kBank / 4 <= kThreads && kBlock / 4 <= kThreads && kWindow / 4 <= kThreads,
              "one 16-byte piece of each scale run per thread");

__device__ __forceinline__ ScalePieces load_scale_pieces(const Segment &seg0, const Segment &seg1,
                                                         int T0, int tb, int te) {
  ScalePieces sp;
  const int e0 = min(te, T0), b1 = max(tb, T0);
  const int i = threadIdx.x;
  sp.i0 = -1;
  sp.i1 = -1;
  sp.k0 = sp.v0 = sp.k1 = sp.v1 = f32x4{0.f, 0.f, 0.f, 0.f};
  if (tb < e0 && i < (e0 - tb) * (kTile8 / 4)) {
    sp.k0 = bitcast<f32x4>(__builtin_amdgcn_raw_buffer_load_b128(seg0.ks, 16 * i, tb * kTile8 * 4, kStream));
    sp.v0 = bitcast<f32x4>(__builtin_amdgcn_raw_buffer_load_b128(seg0.vs, 16 * i, tb * kTile8 * 4, kStream));
    sp.i0 = 4 * i;
  }
  if (b1 < te && i < (te - b1) * (kTile8 / 4)) {
    const int row0 = (b1 - T0) * kTile8;
    sp.k1 = bitcast<f32x4>(__builtin_amdgcn_raw_buffer_load_b128(seg1.ks, 16 * i, row0 * 4, kStream));
    sp.v1 = bitcast<f32x4>(__builtin_amdgcn_raw_buffer_load_b128(seg1.vs, 16 * i, row0 * 4, kStream));
    sp.i1 = (b1 - tb) * kTile8 + 4 * i;
  }
  return sp;
}

__device__ __forceinline__ void store_scale_pieces(const ScalePieces &sp, float *ks_l, float *vs_l) {
  if (sp.i0 >= 0) {
    *reinterpret_cast<f32x4 *>(ks_l + sp.i0) = sp.k0;
    *reinterpret_cast<f32x4 *>(vs_l + sp.i0) = sp.v0;
  }
  if (sp.i1 >= 0) {
    *reinterpret_cast<f32x4 *>(ks_l + sp.i1) = sp.k1;
    *reinterpret_cast<f32x4 *>(vs_l + sp.i1) = sp.v1;
  }
}

// V codes stay E4M3 in LDS: 32 rows of 256 bytes, the 16-byte chunk c of row r at
// chunk position c ^ vswz8(r), so that the 16 rows one half-wave's transposed reads
// touch (rows 4kg..4kg+3 and 16+4kg..16+4kg+3 of two lane groups) hit 16 distinct
// 4-bank positions.
__device__ __forceinline__ int vswz8(int r) { return (r & 7) | (((r >> 4) & 1) << 3); }

// Stage the tile's V codes in the wave's LDS rows (consumes V).
__device__ __forceinline__ void stage_v_fp8(int lane, const uint4 (&V)[8], uint8_t *vl) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    *reinterpret_cast<uint4 *>(vl + r * kDim + (((lane & 15) ^ vswz8(r)) << 4)) = V[i];
  }
}

// Scores of the tile's two 16-key halves (consumes K).  The contraction over the
// head dimension runs in a permuted order that the K loads and the query reads
// share: MFMA (s, h) covers, for lane group kg, dims 64s + 16kg + 8h .. +8.  Lane
// holds, in sc[u], keys 16u + 4kg .. +4 of head hh.
template <bool kInt8>
__device__ __forceinline__ void scores_tile_fp8(int nvalid, int lane, const uint4 (&K)[8],
                                                const float *ks_t, const bf16x8 (&qv)[8],
                                                f32x4 (&sc)[2]) {
  const int kg = lane >> 4;
  sc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  sc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint4 &kw = K[4 * u + s];
        const uint4 kb = h ? q8x8_to_bf16x8<kInt8>(kw.z, kw.w) : q8x8_to_bf16x8<kInt8>(kw.x, kw.y);
        sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(kb), qv[2 * s + h], sc[u],
                                                        0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    sc[u] *= *reinterpret_cast<const f32x4 *>(ks_t + 16 * u + 4 * kg);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (16 * u + 4 * kg + i >= nvalid) sc[u][i] = -INFINITY;
  }
}

// Online-softmax update over the tile's 32 keys and P x V with the keys as a
// 32-long contraction in the order (4kg .. 4kg+3, 16 + 4kg .. 16 + 4kg+3) for
// lane group kg: the P operand comes straight from the score registers and the V
// operand from two transposed 8-byte LDS reads.  A key's numerator weight is its
// rounded probability times its V scale; the denominator sums the rounded
// probabilities.  A key past the end has probability 0 and scale 0.
template <bool kInt8>
__device__ __forceinline__ void accumulate_tile_fp8(const f32x4 (&sc)[2], int lane,
                                                    const uint8_t *vl, const float *vs_t,
                                                    SoftmaxState &st) {
  const int kg = lane >> 4, r = lane & 15;
  const f32x4 vsc[2] = {*reinterpret_cast<const f32x4 *>(vs_t + 4 * kg),
                        *reinterpret_cast<const f32x4 *>(vs_t + 16 + 4 * kg)};
  float mt = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                   fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float m_new = fmaxf(st.m, mt);
  float alpha = 1.f;
  uint32_t pw[4] = {0, 0, 0, 0};
  float psum = 0.f;
  if (m_new != -INFINITY) {
    alpha = __builtin_amdgcn_exp2f(st.m - m_new);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(sc[u][i] - m_new);
      const uint32_t r0 = pack_bf16x2_cvt(e[0], e[1]), r1 = pack_bf16x2_cvt(e[2], e[3]);
      psum += bf16_lo(r0);
      psum += bf16_hi(r0);
      psum += bf16_lo(r1);
      psum += bf16_hi(r1);
      pw[2 * u] = pack_bf16x2_cvt(e[0] * vsc[u][0], e[1] * vsc[u][1]);
      pw[2 * u + 1] = pack_bf16x2_cvt(e[2] * vsc[u][2], e[3] * vsc[u][3]);
    }
  }
  if (__any(m_new != st.m)) {
#pragma unroll
    for (int db = 0; db < 16; ++db) st.acc[db] *= alpha;
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
  const bf16x8 pb = bitcast<bf16x8>(make_uint4(pw[0], pw[1], pw[2], pw[3]));
  // Transposed 8-bit read: within a 16-lane group, lanes 2j and 2j+1 supply the two
  // 8-byte halves of a 16-byte chunk of row K_j, and lane i receives byte i of the
  // eight rows K_0..K_7 -- here the keys 4kg .. 4kg+3, 16 + 4kg .. 16 + 4kg+3, in the
  // order of the P operand -- i.e. dim 16 db + i of those keys, widened to BF16.
  const int j = r >> 1;
  const int key = j < 4 ? 4 * kg + j : 16 + 4 * kg + (j - 4);
  const uint8_t *src = vl + key * kDim + 8 * (r & 1);
  const int sw = vswz8(key);
#pragma unroll
  for (int db = 0; db < 16; ++db) {
    typedef int v2i __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i lds_v2i;
    const v2i c = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(src + ((db ^ sw) << 4)));
    const bf16x8 va = bitcast<bf16x8>(q8x8_to_bf16x8<kInt8>(static_cast<uint32_t>(c[0]),
                                                            static_cast<uint32_t>(c[1])));
    st.acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, st.acc[db], 0, 0, 0);
  }
}

// The 8-bit state decode for either code format (E4M3 or INT8).
template <bool kInt8>
__global__ __launch_bounds__(kThreads, 2) void decode_attn_q8_kernel(DecodeParams a) {
  __shared__ __align__(16) uint8_t v_lds[kWaves][kTile8 * kDim];
  __shared__ __align__(16) uint16_t q_lds[16][kQStride];  // rows 4..15 stay zero
  __shared__ float red_m[kWaves][kHeadsPerGroup], red_l[kWaves][kHeadsPerGroup];
  __shared__ __align__(16) float ks_lds[kMaxScaleKeys], vs_lds[kMaxScaleKeys];
  __shared__ __align__(16) float g_lds[kWaves][kDim];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps tile selection scalar
  int unit, split;
  unit_split_of(blockIdx.x, a.splits, unit, split);
  const int per_branch = a.batch * kGroups;
  const bool anchor = unit < per_branch;
  const int bg = anchor ? unit : unit - per_branch;
  const int b = bg / kGroups, g = bg % kGroups;

  Segment seg0, seg1;
  unit_segments<true>(a, b, g, anchor, seg0, seg1);
  const int T0 = (seg0.n + kTile8 - 1) / kTile8;
  const int T = T0 + (seg1.n + kTile8 - 1) / kTile8;
  const int per = (T + a.splits - 1) / a.splits;
  const int tb = split * per;
  const int te = min(T, tb + per);
  // E4M3: the scales first (the query prologue's barrier publishes them)
  if constexpr (!kInt8) load_scales_fp8(seg0, seg1, T0, tb, te, ks_lds, vs_lds);

  SoftmaxState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int d = 0; d < 16; ++d) st.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint8_t *vl = v_lds[wave];
  uint4 K[8], V[8];
  int t = tb + wave;
  // the query's loads first, then the first tile's (on every path): the prologue
  // waits for the query alone
  const QueryRaw qraw = load_query(a, b, g, anchor, wave, lane);
  {
    const Segment &sg = t < T0 ? seg0 : seg1;
    const int key0 = t < te ? (t < T0 ? t : t - T0) * kTile8 : kNoRows;
    load_v_fp8(sg, key0, lane, V);
    load_k_fp8(sg, key0, lane, K);
  }
  if constexpr (kInt8) {
    // INT8: the scales after the first tile, stored once the query is staged
    const ScalePieces spc = load_scale_pieces(seg0, seg1, T0, tb, te);
    stage_query_raw(a, qraw, a.pos[b], wave, lane, q_lds, g_lds[wave]);
    store_scale_pieces(spc, ks_lds, vs_lds);
    __syncthreads();
  } else {
    stage_query_raw(a, qraw, a.pos[b], wave, lane, q_lds, g_lds[wave]);
  }
  // Query operands in registers: qv[2s + h] holds, for lane (hh, kg), dims
  // 64s + 16kg + 8h .. +8 of head hh (the permuted contraction order).
  bf16x8 qv[8];
  {
    const uint16_t *qrow = &q_lds[0][0] + (lane & 15) * kQStride + 16 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        qv[2 * s + h] = bitcast<bf16x8>(*reinterpret_cast<const uint4 *>(qrow + 64 * s + 8 * h));
  }

  for (; t < te; t += kWaves) {
    const int key0 = (t < T0 ? t : t - T0) * kTile8;
    const int nvalid = (t < T0 ? seg0.n : seg1.n) - key0;
    const int tn = t + kWaves;
    const Segment &nsg = tn < T0 ? seg0 : seg1;
    const int nkey0 = (tn < T0 ? tn : tn - T0) * kTile8;
    stage_v_fp8(lane, V, vl);
    if (tn < te) load_v_fp8(nsg, nkey0, lane, V);
    f32x4 sc[2];
    scores_tile_fp8<kInt8>(nvalid, lane, K, ks_lds + (t - tb) * kTile8, qv, sc);
    if (tn < te) load_k_fp8(nsg, nkey0, lane, K);
    accumulate_tile_fp8<kInt8>(sc, lane, vl, vs_lds + (t - tb) * kTile8, st);
  }

  __syncthreads();
  finish_unit(a, st, reinterpret_cast<float *>(&v_lds[0][0]), red_m, red_l, wave, lane, unit,
              split, anchor, b, g);
}

// Merge the splits of one (branch, sequence, group): 4 waves, one per head.
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeParams a) {
  const int lane = threadIdx.x & 63;
  const int h = threadIdx.x >> 6;
  const int unit = blockIdx.x;
  const int per_branch = a.batch * kGroups;
  const bool anchor = unit < per_branch;
  const int bg = anchor ? unit : unit - per_branch;
  const int b = bg / kGroups, g = bg % kGroups;
  const float *base = a.part + static_cast<size_t>(unit) * a.splits * kHeadsPerGroup * kPartStride +
                      h * kPartStride;
  // Every split's (m, l) and accumulator slice are loaded before any of them is
  // used (the loop is unrolled over the split capacity), so the kernel waits for
  // one round trip to memory rather than one per split or per pass.
  float ms[kMaxSplits], ls[kMaxSplits];
  float4 os[kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    ms[sp] = -INFINITY;
    ls[sp] = 0.f;
    os[sp] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (sp < a.splits) {
      const float *pp = base + static_cast<size_t>(sp) * kHeadsPerGroup * kPartStride;
      const float2 ml = *reinterpret_cast<const float2 *>(pp);
      ms[sp] = ml.x;
      ls[sp] = ml.y;
      os[sp] = *reinterpret_cast<const float4 *>(pp + 4 + 4 * lane);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) M = fmaxf(M, ms[sp]);
  float L = 0.f;
  float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp) {
      const float wt = ms[sp] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[sp] - M);
      L += ls[sp] * wt;
      O.x += os[sp].x * wt;
      O.y += os[sp].y * wt;
      O.z += os[sp].z * wt;
      O.w += os[sp].w * wt;
    }
  }
  const int head = g * kHeadsPerGroup + h;
  uint16_t *o = (anchor ? a.o_rma : a.o_win) + (static_cast<size_t>(b) * kHeads + head) * kDim;
  float *lse = (anchor ? a.lse_rma : a.lse_win) + static_cast<size_t>(b) * kHeads + head;
  uint2 ov = make_uint2(0, 0);
  float lv = -INFINITY;
  if (M != -INFINITY) {
    const float inv = 1.f / L;
    ov.x = pack_bf16x2(O.x * inv, O.y * inv);
    ov.y = pack_bf16x2(O.z * inv, O.w * inv);
    lv = (M + log2f(L)) * kLn2;
  }
  *reinterpret_cast<uint2 *>(o + 4 * lane) = ov;
  if (lane == 0) *lse = lv;
}

}  // namespace rma

using namespace rma;

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool aligned8(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

extern "C" int32_t rma_decode_splits(int32_t batch) {
  if (batch <= 0) return 1;
  // Split each branch's keys until the launch has kMinWorkgroups workgroups.
  const int units = batch * kGroups * 2;
  int s = (kMinWorkgroups + units - 1) / units;
  return s < 1 ? 1 : (s > kMaxSplits ? kMaxSplits : s);
}

extern "C" size_t rma_decode_workspace_bytes(int32_t batch) {
  if (batch <= 0) return 0;
  const int s = rma_decode_splits(batch);
  if (s == 1) return 0;
  return static_cast<size_t>(batch) * kGroups * 2 * s * kHeadsPerGroup * kPartStride * sizeof(float);
}

// Validate the shared arguments and fill the rest of the decode parameters.
template <bool kFp8>
static rma_status prepare_decode(DecodeParams &p, int32_t batch, const uint16_t *q_win,
                                 const uint16_t *q_rma, const rma_norm *norm, uint16_t *o_win,
                                 float *lse_win, uint16_t *o_rma, float *lse_rma, void *workspace,
                                 size_t workspace_bytes) {
  if (!norm || !q_win || !q_rma || !o_win || !lse_win || !o_rma || !lse_rma) return RMA_E_ARG;
  if (batch <= 0 || batch > RMA_MAX_BATCH) return RMA_E_ARG;
  if (!p.win_k || !p.win_v || !p.bank_k || !p.bank_v || !p.pend_k || !p.pend_v || !p.n_bank ||
      !p.n_pend || !p.pos || !norm->gq_win || !norm->gq_rma)
    return RMA_E_ARG;
  if (kFp8 && (!p.win_ks || !p.win_vs || !p.bank_ks || !p.bank_vs || !p.pend_ks || !p.pend_vs))
    return RMA_E_ARG;
  const void *al[] = {p.win_k, p.win_v, p.bank_k, p.bank_v,     p.pend_k,     p.pend_v,
                      q_win,   q_rma,   o_win,    o_rma,        norm->gq_win, norm->gq_rma};
  for (const void *ptr : al)
    if (!aligned16(ptr)) return RMA_E_ALIGN;
  if (kFp8) {
    const void *as[] = {p.win_ks, p.win_vs, p.bank_ks, p.bank_vs, p.pend_ks, p.pend_vs};
    for (const void *ptr : as)
      if (!aligned16(ptr)) return RMA_E_ALIGN;
  }
  const size_t need = rma_decode_workspace_bytes(batch);
  if (need > 0 && (!workspace || workspace_bytes < need)) return RMA_E_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return RMA_E_ALIGN;

  p.q_win = q_win;
  p.q_rma = q_rma;
  p.gq_win = norm->gq_win;
  p.gq_rma = norm->gq_rma;
  p.eps = norm->eps;
  p.rope_ratio = rope_ratio(norm->rope_base);
  p.o_win = o_win;
  p.o_rma = o_rma;
  p.lse_win = lse_win;
  p.lse_rma = lse_rma;
  p.part = static_cast<float *>(workspace);
  p.batch = batch;
  p.splits = rma_decode_splits(batch);
  return RMA_OK;
}

static rma_status launch_merge(const DecodeParams &p, hipStream_t s) {
  if (p.splits > 1) {
    const unsigned units = static_cast<unsigned>(p.batch) * kGroups * 2;
    hipLaunchKernelGGL(decode_merge_kernel, dim3(units), dim3(kMergeThreads), 0, s, p);
    if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  }
  return RMA_OK;
}

// Validate, then launch the decode and the split merge.
// kFp8: an 8-bit state (codes + row scales); kInt8 picks INT8 codes over E4M3.
template <bool kFp8, bool kInt8 = false>
static rma_status launch_decode(DecodeParams &p, int32_t batch, const uint16_t *q_win,
                                const uint16_t *q_rma, const rma_norm *norm, uint16_t *o_win,
                                float *lse_win, uint16_t *o_rma, float *lse_rma, void *workspace,
                                size_t workspace_bytes, void *stream) {
  const rma_status rc = prepare_decode<kFp8>(p, batch, q_win, q_rma, norm, o_win, lse_win, o_rma,
                                             lse_rma, workspace, workspace_bytes);
  if (rc != RMA_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned units = static_cast<unsigned>(batch) * kGroups * 2;
  if constexpr (kFp8)
    hipLaunchKernelGGL(decode_attn_q8_kernel<kInt8>, dim3(units * p.splits), dim3(kThreads), 0, s,
                       p);
  else
    hipLaunchKernelGGL(decode_attn_kernel, dim3(units * p.splits), dim3(kThreads), 0, s, p);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  return launch_merge(p, s);
}

extern "C" rma_status swa_rma_decode_attn(const rma_layer_state *st, int32_t batch,
                                          const uint16_t *q_win, const uint16_t *q_rma,
                                          const rma_norm *norm, uint16_t *o_win, float *lse_win,
                                          uint16_t *o_rma, float *lse_rma, void *workspace,
                                          size_t workspace_bytes, void *stream) {
  if (!st) return RMA_E_ARG;
  DecodeParams p{};
  p.win_k = reinterpret_cast<const uint8_t *>(st->win_k);
  p.win_v = reinterpret_cast<const uint8_t *>(st->win_v);
  p.bank_k = reinterpret_cast<const uint8_t *>(st->bank_k);
  p.bank_v = reinterpret_cast<const uint8_t *>(st->bank_v);
  p.pend_k = reinterpret_cast<const uint8_t *>(st->pend_k);
  p.pend_v = reinterpret_cast<const uint8_t *>(st->pend_v);
  p.n_bank = st->n_bank;
  p.n_pend = st->n_pend;
  p.pos = st->pos;
  return launch_decode<false>(p, batch, q_win, q_rma, norm, o_win, lse_win, o_rma, lse_rma,
                              workspace, workspace_bytes, stream);
}

template <bool kInt8>
static rma_status decode_q8(const rma_layer_state_fp8 *st, int32_t batch, const uint16_t *q_win,
                            const uint16_t *q_rma, const rma_norm *norm, uint16_t *o_win,
                            float *lse_win, uint16_t *o_rma, float *lse_rma, void *workspace,
                            size_t workspace_bytes, void *stream) {
  if (!st) return RMA_E_ARG;
  DecodeParams p{};
  p.win_k = st->win_k;
  p.win_v = st->win_v;
  p.bank_k = st->bank_k;
  p.bank_v = st->bank_v;
  p.pend_k = st->pend_k;
  p.pend_v = st->pend_v;
  p.win_ks = st->win_ks;
  p.win_vs = st->win_vs;
  p.bank_ks = st->bank_ks;
  p.bank_vs = st->bank_vs;
  p.pend_ks = st->pend_ks;
  p.pend_vs = st->pend_vs;
  p.n_bank = st->n_bank;
  p.n_pend = st->n_pend;
  p.pos = st->pos;
  return launch_decode<true, kInt8>(p, batch, q_win, q_rma, norm, o_win, lse_win, o_rma, lse_rma,
                             workspace, workspace_bytes, stream);
}

extern "C" rma_status swa_rma_decode_attn_fp8(const rma_layer_state_fp8 *st, int32_t batch,
                                              const uint16_t *q_win, const uint16_t *q_rma,
                                              const rma_norm *norm, uint16_t *o_win,
                                              float *lse_win, uint16_t *o_rma, float *lse_rma,
                                              void *workspace, size_t workspace_bytes,
                                              void *stream) {
  return decode_q8<false>(st, batch, q_win, q_rma, norm, o_win, lse_win, o_rma, lse_rma,
                          workspace, workspace_bytes, stream);
}

extern "C" rma_status swa_rma_decode_attn_i8(const rma_layer_state_fp8 *st, int32_t batch,
                                             const uint16_t *q_win, const uint16_t *q_rma,
                                             const rma_norm *norm, uint16_t *o_win,
                                             float *lse_win, uint16_t *o_rma, float *lse_rma,
                                             void *workspace, size_t workspace_bytes,
                                             void *stream) {
  return decode_q8<true>(st, batch, q_win, q_rma, norm, o_win, lse_win, o_rma, lse_rma,
                         workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- fused step host
static size_t step_counter_offset(int32_t batch) {
  return (rma_decode_workspace_bytes(batch) + 255) & ~static_cast<size_t>(255);
}

extern "C" size_t rma_step_workspace_bytes(int32_t batch) {
  if (batch <= 0) return 0;
  return step_counter_offset(batch) + static_cast<size_t>(batch) * sizeof(uint32_t);
}

extern "C" rma_status swa_rma_step(const rma_layer_state *st, int32_t batch, const uint16_t *k_win,
                                   const uint16_t *v_win, const uint16_t *k_rma,
                                   const uint16_t *v_rma, const float *score,
                                   const uint16_t *q_win, const uint16_t *q_rma,
                                   const rma_norm *norm, uint16_t *o_win, float *lse_win,
                                   uint16_t *o_rma, float *lse_rma, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  if (!st || !norm || !k_win || !v_win || !k_rma || !v_rma) return RMA_E_ARG;
  if (batch <= 0 || batch > RMA_MAX_BATCH) return RMA_E_ARG;
  if (!st->pend_src || !norm->gk_win || !norm->gk_rma || (score && !st->pend_score))
    return RMA_E_ARG;
  if (!aligned16(norm->gk_win) || !aligned16(norm->gk_rma)) return RMA_E_ALIGN;
  const void *a8[] = {k_win, v_win, k_rma, v_rma};
  for (const void *ptr : a8)
    if (!aligned8(ptr)) return RMA_E_ALIGN;
  if (!workspace || workspace_bytes < rma_step_workspace_bytes(batch)) return RMA_E_WORKSPACE;
  if (!aligned16(workspace)) return RMA_E_ALIGN;

  StepParams sp{};
  DecodeParams &p = sp.d;
  p.win_k = reinterpret_cast<const uint8_t *>(st->win_k);
  p.win_v = reinterpret_cast<const uint8_t *>(st->win_v);
  p.bank_k = reinterpret_cast<const uint8_t *>(st->bank_k);
  p.bank_v = reinterpret_cast<const uint8_t *>(st->bank_v);
  p.pend_k = reinterpret_cast<const uint8_t *>(st->pend_k);
  p.pend_v = reinterpret_cast<const uint8_t *>(st->pend_v);
  p.n_bank = st->n_bank;
  p.n_pend = st->n_pend;
  p.pos = st->pos;
  const rma_status rc = prepare_decode<false>(p, batch, q_win, q_rma, norm, o_win, lse_win, o_rma,
                                              lse_rma, workspace, workspace_bytes);
  if (rc != RMA_OK) return rc;
  sp.win_k = st->win_k;
  sp.win_v = st->win_v;
  sp.pend_k = st->pend_k;
  sp.pend_v = st->pend_v;
  sp.pend_score = st->pend_score;
  sp.pend_src = st->pend_src;
  sp.n_pend = st->n_pend;
  sp.pos = st->pos;
  sp.k_win = k_win;
  sp.v_win = v_win;
  sp.k_rma = k_rma;
  sp.v_rma = v_rma;
  sp.score = score;
  sp.gk_win = norm->gk_win;
  sp.gk_rma = norm->gk_rma;
  sp.done = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + step_counter_offset(batch));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned units = static_cast<unsigned>(batch) * kGroups * 2;
  hipLaunchKernelGGL(decode_step_kernel, dim3(units * p.splits), dim3(kThreads), 0, s, sp);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  return launch_merge(p, s);
}

// ---------------------------------------------------------------- no-alloc decode
// swa_rma_decode_attn for callers that cannot allocate: the split partials go to
// `scratch`, a device array of this library (each GPU holds its own copy until the
// process ends), instead of a caller workspace.  4 MiB covers every batch: only
// batches below 64 split, and the largest of them needs 1008 (unit, split) pairs of
// 4 heads x 260 floats, 4,193,280 bytes (batch 63).
constexpr size_t kScratchBytes = static_cast<size_t>(RMA_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The device address of `scratch` on the device that runs `stream`, resolved once per
// device with that device current.  In host code the array's name is only a host-side
// stand-in; kernels must be given this address.
rma_status scratch_for_stream(hipStream_t stream, void **out) {
  int dev = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return RMA_E_ARG;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = -1;
      if (hipGetDevice(&cur) != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
      if (cur != dev && hipSetDevice(dev) != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev) (void)hipSetDevice(cur);
      if (e != hipSuccess || !p) return (void)hipGetLastError(), RMA_E_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return RMA_OK;
}
}  // namespace

extern "C" rma_status swa_rma_decode_attn_noalloc(const rma_layer_state *st, int32_t batch,
                                                  const uint16_t *q_win, const uint16_t *q_rma,
                                                  const rma_norm *norm, uint16_t *o_win,
                                                  float *lse_win, uint16_t *o_rma, float *lse_rma,
                                                  void *stream) {
  if (!st) return RMA_E_ARG;
  if (batch <= 0 || batch > RMA_MAX_BATCH) return RMA_E_ARG;
  if (rma_decode_workspace_bytes(batch) > kScratchBytes) return RMA_E_WORKSPACE;
  void *ws = nullptr;
  const rma_status rc = scratch_for_stream(static_cast<hipStream_t>(stream), &ws);
  if (rc != RMA_OK) return rc;
  DecodeParams p{};
  p.win_k = reinterpret_cast<const uint8_t *>(st->win_k);
  p.win_v = reinterpret_cast<const uint8_t *>(st->win_v);
  p.bank_k = reinterpret_cast<const uint8_t *>(st->bank_k);
  p.bank_v = reinterpret_cast<const uint8_t *>(st->bank_v);
  p.pend_k = reinterpret_cast<const uint8_t *>(st->pend_k);
  p.pend_v = reinterpret_cast<const uint8_t *>(st->pend_v);
  p.n_bank = st->n_bank;
  p.n_pend = st->n_pend;
  p.pos = st->pos;
  return launch_decode<false>(p, batch, q_win, q_rma, norm, o_win, lse_win, o_rma, lse_rma, ws,
                              kScratchBytes, stream);
}
