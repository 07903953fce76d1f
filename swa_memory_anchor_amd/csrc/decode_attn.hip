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
//    LDS rows and read back transposed as the A operand of
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
#include "rma_device.h"

namespace rma {

constexpr int kTile = 16;
#ifndef RMA_DECODE_WAVES
#define RMA_DECODE_WAVES 4
#endif
constexpr int kWaves = RMA_DECODE_WAVES;  // waves per workgroup, all on one (branch, seq, group)
constexpr int kThreads = 64 * kWaves;
constexpr int kMergeThreads = 64 * kHeadsPerGroup;
static_assert(kWaves >= kHeadsPerGroup, "one wave per head in the query prologue and epilogue");
constexpr int kVStride = kDim + 8;  // LDS row stride of a V tile, in elements (528 B)
constexpr int kPartStride = 4 + kDim;
constexpr int kMaxSplits = 20;
#ifndef RMA_DECODE_MIN_WGS
#define RMA_DECODE_MIN_WGS 512
#endif
// Split each branch only until a launch has two workgroups per CU (256 CUs):
// more, smaller workgroups measured slower at batch 64 and 512 (per-workgroup
// prologue, partial writes and the merge launch cost more than they balance).
constexpr int kMinWorkgroups = RMA_DECODE_MIN_WGS;
constexpr float kQScale = 1.4426950408889634f / 16.0f;  // log2(e) / sqrt(256)
constexpr float kLn2 = 0.69314718055994531f;
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
// size is the valid byte count: rows past the end read as zero.
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

// Bytes of one K/V row.
template <bool kFp8>
constexpr int kRowBytes = kFp8 ? kDim : 2 * kDim;

// Bytes of the scales of n rows, rounded up to whole groups of four rows.
__device__ __forceinline__ int scale_bytes(int n) { return ((n + 3) & ~3) * 4; }

// Issue the loads of one 16-key tile starting at row key0 of a segment: K as MFMA
// A operands (lane: row key0 + lane%16, dims 32s + 8(lane/16) .. +8), V as row
// chunks (lane: row key0 + 2i + lane/32, dims 8(lane%32) .. +8).  BF16 rows fill
// all of each uint4; FP8 rows only .x and .y (8 codes).  The FP8 variant also
// loads the scales of the lane's four score keys (key0 + 4(lane/16) + 0..3).
template <bool kFp8>
__device__ __forceinline__ void load_tile(const Segment &sg, int key0, int lane, uint4 (&K)[8],
                                          uint4 (&V)[8], f32x4 &ks, f32x4 &vs) {
  constexpr int RB = kRowBytes<kFp8>;
  constexpr int EB = kFp8 ? 1 : 2;  // bytes per element
  const int hh = lane & 15, kg = lane >> 4;
  const int koff = hh * RB + kg * 8 * EB;
  const int voff = (lane >> 5) * RB + (lane & 31) * 8 * EB;
  const int soff = key0 * RB;
  if constexpr (kFp8) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b64(sg.k, koff + 32 * s, soff, kStream);
      K[s].x = w[0];
      K[s].y = w[1];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b64(sg.v, voff + 2 * RB * i, soff, kStream);
      V[i].x = w[0];
      V[i].y = w[1];
    }
    ks = bitcast<f32x4>(__builtin_amdgcn_raw_buffer_load_b128(sg.ks, 16 * kg, key0 * 4, kStream));
    vs = bitcast<f32x4>(__builtin_amdgcn_raw_buffer_load_b128(sg.vs, 16 * kg, key0 * 4, kStream));
  } else {
    (void)ks;
    (void)vs;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      K[s] = bitcast<uint4>(__builtin_amdgcn_raw_buffer_load_b128(sg.k, koff + 64 * s, soff, kStream));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      V[i] = bitcast<uint4>(
          __builtin_amdgcn_raw_buffer_load_b128(sg.v, voff + 2 * RB * i, soff, kStream));
  }
}

// Eight E4M3 codes -> eight BF16 values (every E4M3 value is exact in BF16).
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  auto hi16 = [](float x, float y) {
    return (__float_as_uint(x) >> 16) | (__float_as_uint(y) & 0xffff0000u);
  };
  return make_uint4(hi16(a[0], a[1]), hi16(b[0], b[1]), hi16(c[0], c[1]), hi16(d[0], d[1]));
}

struct SoftmaxState {
  float m, l;
  f32x4 acc[16];
};

// Stage V in LDS and form the scores of one tile (consumes K and V).  FP8 rows are
// widened to BF16 on the way; a key's score is multiplied by its K scale.
template <bool kFp8>
__device__ __forceinline__ f32x4 scores_tile(int nvalid, int lane, const uint4 (&K)[8],
                                             const uint4 (&V)[8], const f32x4 &ks,
                                             const uint16_t *ql, uint16_t *vl) {
  const int hh = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint4 *>(vl + (2 * i + (lane >> 5)) * kVStride + 8 * (lane & 31)) =
        kFp8 ? fp8x8_to_bf16x8(V[i].x, V[i].y) : V[i];
  // D[key][head] = sum_d K[key][d] * qhat[head][d]; the B operand is the staged
  // query block (head hh; rows >= 4 are zero).  Lane holds keys 4kg..4kg+3 of head hh.
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
  const uint16_t *qrow = ql + hh * kDim + 8 * kg;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const bf16x8 qv = bitcast<bf16x8>(*reinterpret_cast<const uint4 *>(qrow + 32 * s));
    const uint4 kv = kFp8 ? fp8x8_to_bf16x8(K[s].x, K[s].y) : K[s];
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(kv), qv, sc, 0, 0, 0);
  }
  if constexpr (kFp8) sc *= ks;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (4 * kg + i >= nvalid) sc[i] = -INFINITY;
  return sc;
}

// Online-softmax update and P x V for one tile whose V rows are staged in LDS.
// The FP8 variant weighs each value row by its scale in the numerator (the
// denominator sums the unscaled probabilities).
template <bool kFp8>
__device__ __forceinline__ void accumulate_tile(f32x4 sc, int lane, const uint16_t *vl,
                                                const f32x4 &vsc, SoftmaxState &st) {
  const int hh = lane & 15, kg = lane >> 4;
  float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float m_new = fmaxf(st.m, mt);
  float alpha = 1.f;
  uint32_t pw0 = 0, pw1 = 0;
  float psum = 0.f;
  if (m_new != -INFINITY) {
    alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    const float e0 = __builtin_amdgcn_exp2f(sc[0] - m_new);
    const float e1 = __builtin_amdgcn_exp2f(sc[1] - m_new);
    const float e2 = __builtin_amdgcn_exp2f(sc[2] - m_new);
    const float e3 = __builtin_amdgcn_exp2f(sc[3] - m_new);
    const uint32_t p0 = f32_to_bf16(e0), p1 = f32_to_bf16(e1);
    const uint32_t p2 = f32_to_bf16(e2), p3 = f32_to_bf16(e3);
    // the denominator uses the same rounded weights as the numerator
    psum = (bf16_to_f32(p0) + bf16_to_f32(p1)) + (bf16_to_f32(p2) + bf16_to_f32(p3));
    if constexpr (kFp8) {
      pw0 = f32_to_bf16(e0 * vsc[0]) | (f32_to_bf16(e1 * vsc[1]) << 16);
      pw1 = f32_to_bf16(e2 * vsc[2]) | (f32_to_bf16(e3 * vsc[3]) << 16);
    } else {
      (void)vsc;
      pw0 = p0 | (p1 << 16);
      pw1 = p2 | (p3 << 16);
    }
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
  const s16x4 pb = bitcast<s16x4>(make_uint2(pw0, pw1));
  // D[dim][head] += sum_key V[key][dim] * P[head][key].  This wave's LDS reads
  // follow its own writes in scores_tile (LDS runs a wave's operations in order).
#pragma unroll
  for (int db = 0; db < 16; ++db) {
    const uint16_t *col = vl + db * 16 + hh + 4 * kg * kVStride;
    const uint32_t w0 = col[0] | (static_cast<uint32_t>(col[kVStride]) << 16);
    const uint32_t w1 = col[2 * kVStride] | (static_cast<uint32_t>(col[3 * kVStride]) << 16);
    const s16x4 va = bitcast<s16x4>(make_uint2(w0, w1));
    st.acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, st.acc[db] * alpha, 0, 0, 0);
  }
}

template <bool kFp8>
__global__ __launch_bounds__(kThreads, 2) void decode_attn_kernel(DecodeParams a) {
  __shared__ __align__(16) uint16_t v_lds[kWaves][kTile * kVStride];
  __shared__ __align__(16) uint16_t q_lds[16][kDim];  // rows 4..15 stay zero
  __shared__ float red_m[kWaves][kHeadsPerGroup], red_l[kWaves][kHeadsPerGroup];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int split = blockIdx.x % a.splits;
  const int unit = blockIdx.x / a.splits;
  const int per_branch = a.batch * kGroups;
  const bool anchor = unit < per_branch;  // anchor units first: they are the longer ones
  const int bg = anchor ? unit : unit - per_branch;
  const int b = bg / kGroups, g = bg % kGroups;

  const int p = a.pos[b];
  Segment seg0, seg1;
  const size_t sgi = static_cast<size_t>(b) * kGroups + g;
  constexpr int RB = kRowBytes<kFp8>;
  if (anchor) {
    const int nb = min(max(a.n_bank[b], 0), kBank);
    const int np = min(max(a.n_pend[b], 0), kBlock);
    seg0.k = make_rsrc(a.bank_k + sgi * kBank * RB, nb * RB);
    seg0.v = make_rsrc(a.bank_v + sgi * kBank * RB, nb * RB);
    seg0.n = nb;
    seg1.k = make_rsrc(a.pend_k + sgi * kBlock * RB, np * RB);
    seg1.v = make_rsrc(a.pend_v + sgi * kBlock * RB, np * RB);
    seg1.n = np;
    if constexpr (kFp8) {
      // scales are read four keys at a time: the range covers whole quads (the
      // arrays hold a multiple of four rows), and keys past n are masked
      seg0.ks = make_rsrc(a.bank_ks + sgi * kBank, scale_bytes(nb));
      seg0.vs = make_rsrc(a.bank_vs + sgi * kBank, scale_bytes(nb));
      seg1.ks = make_rsrc(a.pend_ks + sgi * kBlock, scale_bytes(np));
      seg1.vs = make_rsrc(a.pend_vs + sgi * kBlock, scale_bytes(np));
    }
  } else {
    const int nw = min(max(p + 1, 0), kWindow);
    seg0.k = make_rsrc(a.win_k + sgi * kWindow * RB, nw * RB);
    seg0.v = make_rsrc(a.win_v + sgi * kWindow * RB, nw * RB);
    seg0.n = nw;
    if constexpr (kFp8) {
      seg0.ks = make_rsrc(a.win_ks + sgi * kWindow, scale_bytes(nw));
      seg0.vs = make_rsrc(a.win_vs + sgi * kWindow, scale_bytes(nw));
    }
    seg1 = seg0;
    seg1.n = 0;
  }
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
  f32x4 ks, vs;
  int t = tb + wave;
  // The first tile's loads do not depend on the query: issue them before the
  // query prologue so its latency overlaps the norm and rotary work.
  if (t < te)
    load_tile<kFp8>(t < T0 ? seg0 : seg1, (t < T0 ? t : t - T0) * kTile, lane, K, V, ks, vs);

  // Query prep: wave w < 4 normalises, rotates and scales head 4g + w.
  if (wave < kHeadsPerGroup) {
    const uint16_t *q = (anchor ? a.q_rma : a.q_win) +
                        (static_cast<size_t>(b) * kHeads + g * kHeadsPerGroup + wave) * kDim;
    const uint2 raw = *reinterpret_cast<const uint2 *>(q + 4 * lane);
    float x[4] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y)};
    float c, sn;
    rope_cos_sin(a.rope_ratio, p, lane, c, sn);
    norm_rope_head(x, anchor ? a.gq_rma : a.gq_win, a.eps, c, sn, lane);
    uint2 o;
    o.x = pack_bf16x2(x[0] * kQScale, x[1] * kQScale);
    o.y = pack_bf16x2(x[2] * kQScale, x[3] * kQScale);
    *reinterpret_cast<uint2 *>(&q_lds[wave][4 * lane]) = o;
  }
  for (int i = threadIdx.x; i < 12 * kDim / 4; i += kThreads)
    reinterpret_cast<uint2 *>(&q_lds[kHeadsPerGroup][0])[i] = make_uint2(0, 0);
  __syncthreads();

  for (; t < te; t += kWaves) {
    const int key0 = (t < T0 ? t : t - T0) * kTile;
    const int nvalid = (t < T0 ? seg0.n : seg1.n) - key0;
    const f32x4 sc = scores_tile<kFp8>(nvalid, lane, K, V, ks, &q_lds[0][0], vl);
    // this tile's value scales, taken before the next tile's loads; a key past the
    // end weighs 0 whatever its slot holds (its probability is 0, and 0 * inf is NaN)
    f32x4 vsc;
#pragma unroll
    for (int i = 0; i < 4; ++i) vsc[i] = 4 * (lane >> 4) + i < nvalid ? vs[i] : 0.f;
    // K and V are consumed: the next tile's loads fly while this one accumulates.
    const int tn = t + kWaves;
    if (tn < te)
      load_tile<kFp8>(tn < T0 ? seg0 : seg1, (tn < T0 ? tn : tn - T0) * kTile, lane, K, V, ks, vs);
    accumulate_tile<kFp8>(sc, lane, vl, vsc, st);
  }

  // Sum the denominators of the four lanes that share a head.
  float l_tot = st.l + __shfl_xor(st.l, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);

  __syncthreads();  // every wave is done with its V rows; reuse them for the merge
  float *macc = reinterpret_cast<float *>(&v_lds[0][0]);  // [wave][head][256]
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

// Validate the shared arguments and launch the decode (and the split merge).
template <bool kFp8>
static rma_status launch_decode(DecodeParams &p, int32_t batch, const uint16_t *q_win,
                                const uint16_t *q_rma, const rma_norm *norm, uint16_t *o_win,
                                float *lse_win, uint16_t *o_rma, float *lse_rma, void *workspace,
                                size_t workspace_bytes, void *stream) {
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned units = static_cast<unsigned>(batch) * kGroups * 2;
  hipLaunchKernelGGL(decode_attn_kernel<kFp8>, dim3(units * p.splits), dim3(kThreads), 0, s, p);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  if (p.splits > 1) {
    hipLaunchKernelGGL(decode_merge_kernel, dim3(units), dim3(kMergeThreads), 0, s, p);
    if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  }
  return RMA_OK;
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

extern "C" rma_status swa_rma_decode_attn_fp8(const rma_layer_state_fp8 *st, int32_t batch,
                                              const uint16_t *q_win, const uint16_t *q_rma,
                                              const rma_norm *norm, uint16_t *o_win,
                                              float *lse_win, uint16_t *o_rma, float *lse_rma,
                                              void *workspace, size_t workspace_bytes,
                                              void *stream) {
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
  return launch_decode<true>(p, batch, q_win, q_rma, norm, o_win, lse_win, o_rma, lse_rma,
                             workspace, workspace_bytes, stream);
}
