// Decode step of the Gated DeltaNet (GDN) layers on gfx950.
//
// fluxbbs.com "EdgeRock-4B 开源：72 MiB 固定 KV，AIME 82.9 分": 24 GDN layers carry a
// fixed-size recurrent matrix per value head (section "架构：递归、局部窗口与记忆锚点
// 三件套": 16 key heads, 32 value heads, convolution width 4), held in FP16 when
// batched and FP32 at batch 1 (section "72 MiB 是怎么算出来的").  The step is the
// gated delta rule (see gdn.h for the conventions and the head-width reading).
//
// Bound: HBM.  Per (sequence, layer) the step reads and writes the 32 value heads'
// 128 x 128 matrices (2 MiB in FP16) against about 6 flop per element, so the
// kernel is built to move each matrix byte once:
//  * one workgroup (4 waves) per (sequence, value head, column slice); a thread
//    owns 8 consecutive value columns of a few key rows and loads them with
//    16-byte non-temporal loads, issued before anything else;
//  * meanwhile the workgroup forms the head's convolution outputs (q and k of
//    its key head, v of its value head), their L2 norms, k.q and the two gates;
//  * the new matrix follows from the old one in one pass: with S' = aS + k u^T
//    and u = b (v - a S^T k), the output S'^T q = a S^T q + u (k.q) needs the
//    same column sums S^T k and S^T q, reduced over the key rows (shuffles, then
//    LDS across the waves); each thread then writes its elements of S' once;
//  * a column slice narrower than the head spreads a small batch over more
//    workgroups (the column sums do not cross columns).
#include <hip/hip_runtime.h>

#include "gdn.h"
#include "rma_device.h"

// No implicit fused multiply-adds in this file: every fma is written out, so the
// decode step and the chunked prefill, which repeat the same per-token arithmetic
// in different code, round identically.
#pragma clang fp contract(off)

namespace gdn {

constexpr int kKH = GDN_K_HEADS;
constexpr int kVH = GDN_V_HEADS;
constexpr int kD = GDN_HEAD_DIM;
constexpr int kConv = GDN_CONV;
constexpr int kCD = GDN_CONV_DIM;
constexpr int kKeyDim = kKH * kD;  // channel offset of k
constexpr int kValOff = 2 * kKeyDim;  // channel offset of v
constexpr int kThreads = 256;
constexpr float kL2Eps = 1e-6f;
// Value columns per workgroup for batches of 16 and more (128: one workgroup per
// head).
#ifndef RMA_GDN_WIDE_COLS
#define RMA_GDN_WIDE_COLS 128
#endif

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct Params {
  void *S;
  uint16_t *conv;
  const uint16_t *x;
  const float *a, *b;
  const int32_t *pos;
  const float *conv_w, *a_log, *dt_bias;
  uint16_t *o;
};

__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// An FP32 result rounded to FP16 (nearest even).  The empty asm hides where x came
// from, so the compiler cannot merge the conversion into the fma that produced it
// (v_fma_mix*_f16 round the exact product-sum once, not the FP32 result): every
// matrix element is rounded to FP32 by its fma and then to FP16, in both kernels.
__device__ __forceinline__ _Float16 to_f16(float x) {
  asm("" : "+v"(x));
  return static_cast<_Float16>(x);
}

// Lane moves for the reductions below: a DPP move within 16-lane rows (kCtrl is the
// DPP control: 0xB1 and 0x4E exchange lanes 1 and 2 apart inside groups of four,
// 0x141 mirrors each half row, 0x140 each row, 0x12n rotates a row by n lanes),
// and the two gfx950 swaps between 16-lane rows and between 32-lane halves.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// The sum over the wave, the same value in every lane: lanes 1 and 2 apart inside
// groups of four, then the other four of each eight, the other eight of each row
// (the row mirrors), then across rows and halves (lane swaps).  No LDS round trips.
__device__ __forceinline__ float wave_total(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                     false);
    v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                   false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// One wave's column sums: the partials pk[j] (S^T k) and pq[j] (S^T q) of columns
// 8c..8c+7 are added over the lanes that share the chunk c (lanes kChunks apart),
// and the totals go to red[0][8c + j] and red[1][8c + j].  The pairs are those of
// a butterfly over lane offsets kChunks, 2 kChunks, ... (smallest first): offsets 4
// and 8 by rotating 16-lane rows (with 4 chunks; the sum is complete in the lanes
// whose row position is 12..15), 16 and 32 by v_permlane16_swap and
// v_permlane32_swap, two values per swap.
template <int kChunks, int kCW>
__device__ __forceinline__ void column_sums(float (&pk)[8], float (&pq)[8], float (*red)[kCW],
                                            int lane) {
  static_assert(kChunks == 4 || kChunks == 16, "column chunks per slice");
  if constexpr (kChunks == 4) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pk[j] += dpp_mov<0x124>(pk[j]);
      pq[j] += dpp_mov<0x124>(pq[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pk[j] += dpp_mov<0x128>(pk[j]);
      pq[j] += dpp_mov<0x128>(pq[j]);
    }
  }
  float pv[16], r1[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pv[j] = pk[j];
    pv[8 + j] = pq[j];
  }
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(pv[2 * n]),
                                                     __float_as_uint(pv[2 * n + 1]), false, false);
    r1[n] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  // lane l of sum n: value 4n + l / 16 (S^T k for 0..7, then S^T q) of chunk l % kChunks
  const int cl = lane & (kChunks - 1), sub = lane >> 4;
  const bool writer = kChunks == 16 || ((lane >> 2) & 3) == 3;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(r1[2 * n]),
                                                     __float_as_uint(r1[2 * n + 1]), false, false);
    const int m = 4 * n + sub;
    if (writer) red[m >> 3][8 * cl + (m & 7)] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
}

// The inputs of one channel: all four ring slots (loaded without waiting for the
// position, which only selects among them), the current input and the taps.
struct ConvIn {
  uint16_t r[kConv];
  uint16_t x;
  float4 w;
};

__device__ __forceinline__ ConvIn conv_load(const Params &pr, const uint16_t *ring,
                                            const uint16_t *xb, int ch) {
  ConvIn c;
#pragma unroll
  for (int j = 0; j < kConv; ++j) c.r[j] = ring[j * kCD + ch];
  c.x = xb[ch];
  c.w = *reinterpret_cast<const float4 *>(pr.conv_w + 4 * ch);
  return c;
}

// Ring slot i (0..3) by selects, so the four values stay in registers.
__device__ __forceinline__ float ring_at(const ConvIn &c, int i) {
  const uint16_t lo = (i & 1) ? c.r[1] : c.r[0];
  const uint16_t hi = (i & 1) ? c.r[3] : c.r[2];
  return bf16f((i & 2) ? hi : lo);
}

// SiLU of the width-4 causal convolution at position p: taps 0..2 take the inputs
// of positions p-3..p-1 (ring slots (p-3..p-1) mod 4), tap 3 the current input.
__device__ __forceinline__ float conv_silu(const ConvIn &c, int p) {
  float acc = c.w.x * ring_at(c, (p - 3) & 3);
  acc = fmaf(c.w.y, ring_at(c, (p - 2) & 3), acc);
  acc = fmaf(c.w.z, ring_at(c, (p - 1) & 3), acc);
  acc = fmaf(c.w.w, bf16f(c.x), acc);
  return acc / (1.f + expf(-acc));
}

// Eight loaded matrix elements (one 16-byte vector of FP16, two of FP32) as floats.
template <int kVec>
__device__ __forceinline__ void widen(const f32x4_t (&v)[kVec], float (&e)[8]) {
  if constexpr (kVec == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      e[j] = v[0][j];
      e[4 + j] = v[1][j];
    }
  } else {
    const f16x8 hv = __builtin_bit_cast(f16x8, v[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = static_cast<float>(hv[j]);
  }
}

template <bool kF32, int kCW>
__global__ __launch_bounds__(kThreads) void gdn_decode_kernel(Params pr) {
  constexpr int kChunks = kCW / 8;         // 8-column chunks per slice
  constexpr int kRG = kThreads / kChunks;  // row groups
  constexpr int kRows = kD / kRG;          // key rows per thread
  constexpr int kSlices = kD / kCW;
  constexpr int kWaves = kThreads / 64;
  __shared__ float q_s[kD], k_s[kD], v_s[kD];
  __shared__ float red[kWaves][2][kCW];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int slice = blockIdx.x % kSlices;
  const int bh = blockIdx.x / kSlices;
  const int b = bh / kVH, h = bh % kVH, kh = h / (kVH / kKH);
  const int c = t % kChunks, rg = t / kChunks;
  const int col = slice * kCW + 8 * c;  // first value column of this thread
  const size_t head = static_cast<size_t>(bh) * kD * kD;

  // 1. this thread's elements of the matrix: rows rg + kRG i, columns col .. col+7
  constexpr int kVec = kF32 ? 2 : 1;  // 16-byte vectors per 8 elements
  f32x4_t raw[kRows][kVec];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const size_t e = head + static_cast<size_t>(rg + kRG * i) * kD + col;
    if constexpr (kF32) {
      const f32x4_t *src = reinterpret_cast<const f32x4_t *>(static_cast<const float *>(pr.S) + e);
      raw[i][0] = __builtin_nontemporal_load(src);
      raw[i][1] = __builtin_nontemporal_load(src + 1);
    } else {
      const f32x4_t *src =
          reinterpret_cast<const f32x4_t *>(static_cast<const _Float16 *>(pr.S) + e);
      raw[i][0] = __builtin_nontemporal_load(src);
    }
  }

  // 2. convolution outputs of the channels this head reads; the ring keeps x.  All
  // of the step's small loads are issued together, before any of them is used.
  const uint16_t *xb = pr.x + static_cast<size_t>(b) * kCD;
  uint16_t *ring = pr.conv + static_cast<size_t>(b) * kConv * kCD;
  const int ch0 = t < kD ? kh * kD + t : kKeyDim + kh * kD + (t - kD);  // q, then k
  const int cv = kValOff + h * kD + (t & (kD - 1));
  const ConvIn in0 = conv_load(pr, ring, xb, ch0);
  ConvIn in1;
  if (t < kD) in1 = conv_load(pr, ring, xb, cv);
  const int p = pr.pos[b];
  const float za = pr.a[b * kVH + h] + pr.dt_bias[h];
  const float zb = pr.b[b * kVH + h];
  const float a_log = pr.a_log[h];
  uint16_t *slot = ring + (p & 3) * kCD;
  const float y0 = conv_silu(in0, p);
  if (t < kD) {
    q_s[t] = y0;
    v_s[t] = conv_silu(in1, p);
    if (slice == 0) slot[cv] = in1.x;
  } else {
    k_s[t - kD] = y0;
  }
  if (slice == 0 && (h & 1) == 0) slot[ch0] = in0.x;
  __syncthreads();

  // L2 norms and k.q (every wave forms them for itself), gates
  const float q0 = q_s[lane], q1 = q_s[lane + 64], k0 = k_s[lane], k1 = k_s[lane + 64];
  const float sq = wave_total(q0 * q0 + q1 * q1);
  const float sk = wave_total(k0 * k0 + k1 * k1);
  const float sqk = wave_total(q0 * k0 + q1 * k1);
  const float iq = (1.f / sqrtf(sq + kL2Eps)) * 0.08838834764831845f;  // 1/sqrt(128)
  const float ik = 1.f / sqrtf(sk + kL2Eps);
  const float kq = sqk * iq * ik;
  const float softplus = fmaxf(za, 0.f) + log1pf(expf(-fabsf(za)));
  const float alpha = expf(-expf(a_log) * softplus);
  const float eb = expf(-fabsf(zb));
  const float beta = zb >= 0.f ? 1.f / (1.f + eb) : eb / (1.f + eb);

  // 3. column sums S^T k and S^T q over this thread's rows, then over all rows.  The
  // elements stay in their loaded (packed) form and are widened again for the
  // update, which keeps the register count, and with it the workgroups per CU
  // that hide the memory latency, up.
  float pk[8], pq[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) pk[j] = pq[j] = 0.f;
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int r = rg + kRG * i;
    const float kr = k_s[r] * ik, qr = q_s[r] * iq;
    float e[8];
    widen(raw[i], e);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pk[j] = fmaf(e[j], kr, pk[j]);
      pq[j] = fmaf(e[j], qr, pq[j]);
    }
  }
  column_sums<kChunks, kCW>(pk, pq, red[wave], lane);
  __syncthreads();

  // 4. u, the output, and the new matrix
  float u[8], o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float tk = 0.f, tq = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      tk += red[w][0][8 * c + j];
      tq += red[w][1][8 * c + j];
    }
    u[j] = beta * (v_s[col + j] - alpha * tk);
    o[j] = fmaf(alpha, tq, u[j] * kq);
  }
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int r = rg + kRG * i;
    const float kr = k_s[r] * ik;
    const size_t e = head + static_cast<size_t>(r) * kD + col;
    float sv[8];
    widen(raw[i], sv);
    if constexpr (kF32) {
      f32x4_t lo, hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo[j] = fmaf(alpha, sv[j], kr * u[j]);
        hi[j] = fmaf(alpha, sv[4 + j], kr * u[4 + j]);
      }
      f32x4_t *dst = reinterpret_cast<f32x4_t *>(static_cast<float *>(pr.S) + e);
      __builtin_nontemporal_store(lo, dst);
      __builtin_nontemporal_store(hi, dst + 1);
    } else {
      f16x8 hv;
#pragma unroll
      for (int j = 0; j < 8; ++j) hv[j] = to_f16(fmaf(alpha, sv[j], kr * u[j]));
      __builtin_nontemporal_store(__builtin_bit_cast(f32x4_t, hv),
                                  reinterpret_cast<f32x4_t *>(static_cast<_Float16 *>(pr.S) + e));
    }
  }
  if (rg == 0) {
    uint4 ov;
    ov.x = rma::pack_bf16x2(o[0], o[1]);
    ov.y = rma::pack_bf16x2(o[2], o[3]);
    ov.z = rma::pack_bf16x2(o[4], o[5]);
    ov.w = rma::pack_bf16x2(o[6], o[7]);
    *reinterpret_cast<uint4 *>(pr.o + static_cast<size_t>(bh) * kD + col) = ov;
  }
}

// ---------------------------------------------------------------- chunked prefill
// n_tokens successive decode steps of one sequence's head in one workgroup: the
// column slice of the matrix stays in registers (as FP32 values, rounded to the
// storage type after every token, exactly as a stored and reloaded matrix would
// be), and each channel's convolution history (the previous three inputs) in the
// registers of the thread that owns the channel.  Every token runs the decode
// step's arithmetic in the same order, so the results are those of n_tokens
// gdn_decode_step calls, bit for bit.  The ring is read here (history before the
// chunk) and written by the launch that follows (the chunk's last inputs), so no
// workgroup overwrites slots another still has to read.
struct PrefillParams {
  void *S;
  const uint16_t *conv;
  const uint16_t *x;       // [B][T][8192]
  const float *a, *b;      // [B][T][32]
  const int32_t *pos;      // [B]: position of the chunk's first token
  const float *conv_w, *a_log, *dt_bias;
  uint16_t *o;             // [B][T][32][128]
  int n_tokens;
};

// The convolution history of one channel at the chunk's start: the inputs of
// positions p0-3 .. p0-1 (ring slots), oldest first.
__device__ __forceinline__ void history_load(const uint16_t *ring, int ch, int p0, uint16_t (&h)[3]) {
#pragma unroll
  for (int j = 0; j < 3; ++j) h[j] = ring[((p0 - 3 + j) & 3) * kCD + ch];
}

// SiLU of the width-4 causal convolution of one channel: taps 0..2 on the history
// (positions p-3 .. p-1), tap 3 on the current input (the decode step's order).
__device__ __forceinline__ float conv_silu_hist(const float4 &w, const uint16_t (&h)[3], uint16_t x) {
  float acc = w.x * bf16f(h[0]);
  acc = fmaf(w.y, bf16f(h[1]), acc);
  acc = fmaf(w.z, bf16f(h[2]), acc);
  acc = fmaf(w.w, bf16f(x), acc);
  return acc / (1.f + expf(-acc));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fmaf(a, h, c) for the FP16 value h held in the low (kHi false) or high half of
// the packed register p, as one v_fma_mix_f32: the instruction widens h exactly
// and rounds the fma to FP32 once, as fmaf does.  
template <bool kHi>
__device__ __forceinline__ float fma_f16(float a, uint32_t p, float c) {
  float d;
  if constexpr (kHi)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
        : "=v"(d)
        : "v"(a), "v"(p), "v"(c));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(p), "v"(c));
  return d;
}

// Two FP32 values rounded to FP16 (nearest even) and packed, lo in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  uint32_t d;
  asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(d) : "v"(lo), "v"(hi));
  return d;
}

// Tokens whose inputs (convolutions, norms, gates) are prepared together before
// the recurrence walks them: none of these depend on the matrix, so they are formed
// in parallel over the group's tokens instead of inside the serial token loop.
constexpr int kGroup = 16;

template <bool kF32, int kCW>
__global__ __launch_bounds__(kThreads) void gdn_prefill_kernel(PrefillParams pr) {
  constexpr int kChunks = kCW / 8;
  constexpr int kRG = kThreads / kChunks;
  constexpr int kRows = kD / kRG;
  constexpr int kSlices = kD / kCW;
  constexpr int kWaves = kThreads / 64;
  constexpr int kG = kGroup;
  // per token of the group: q and k scaled by their inverse norms (q also by
  // 1/sqrt(128)), v, and the scalars alpha, beta and k.q
  __shared__ float qn_s[kG][kD], kn_s[kG][kD], v_s[kG][kD];
  __shared__ float al_s[kG], be_s[kG], kq_s[kG];
  __shared__ float red[kWaves][2][kCW];
  __shared__ float u_s[kCW];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int slice = blockIdx.x % kSlices;
  const int bh = blockIdx.x / kSlices;
  const int b = bh / kVH, h = bh % kVH, kh = h / (kVH / kKH);
  const int c = t % kChunks, rg = t / kChunks;
  const int col = slice * kCW + 8 * c;
  const size_t head = static_cast<size_t>(bh) * kD * kD;
  const int T = pr.n_tokens;

  // the matrix slice in its storage type: FP32 values, or FP16 pairs packed in
  // 32-bit words (columns 2k and 2k+1 of a row in word k), which feed the FP32
  // arithmetic through v_fma_mix_f32 with no separate widening
  float sf[kF32 ? kRows : 1][8];
  uint32_t sw[kF32 ? 1 : kRows][4];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const size_t e = head + static_cast<size_t>(rg + kRG * i) * kD + col;
    if constexpr (kF32) {
      const f32x4_t *src = reinterpret_cast<const f32x4_t *>(static_cast<const float *>(pr.S) + e);
      const f32x4_t lo = __builtin_nontemporal_load(src), hi = __builtin_nontemporal_load(src + 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sf[i][j] = lo[j];
        sf[i][4 + j] = hi[j];
      }
    } else {
      const u32x4 w = __builtin_bit_cast(
          u32x4, __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(
                     static_cast<const _Float16 *>(pr.S) + e)));
#pragma unroll
      for (int k = 0; k < 4; ++k) sw[i][k] = w[k];
    }
  }

  // channels: threads t < 128 own q channel t of the key head and v channel t of
  // the value head; threads t >= 128 own k channel t - 128
  const int p0 = pr.pos[b];
  const uint16_t *ring = pr.conv + static_cast<size_t>(b) * kConv * kCD;
  const int ch0 = t < kD ? kh * kD + t : kKeyDim + kh * kD + (t - kD);
  const int cv = kValOff + h * kD + (t & (kD - 1));
  const float4 w0 = *reinterpret_cast<const float4 *>(pr.conv_w + 4 * ch0);
  const float4 w1 = *reinterpret_cast<const float4 *>(pr.conv_w + 4 * cv);
  uint16_t h0[3], h1[3];
  history_load(ring, ch0, p0, h0);
  history_load(ring, cv, p0, h1);
  const float a_log = pr.a_log[h], dtb = pr.dt_bias[h];

  for (int base = 0; base < T; base += kG) {
    const int G = min(kG, T - base);
    const size_t tok0 = static_cast<size_t>(b) * T + base;

    // 1. the group's inputs, then each channel's convolutions in token order
    uint16_t xa[kG], xv[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      if (g < G) {
        const uint16_t *xb = pr.x + (tok0 + g) * kCD;
        xa[g] = xb[ch0];
        xv[g] = t < kD ? xb[cv] : uint16_t(0);
      }
    }
    float ra = 0.f, rb = 0.f;  // gate inputs of token `lane`
    if (lane < G) {
      ra = pr.a[(tok0 + lane) * kVH + h];
      rb = pr.b[(tok0 + lane) * kVH + h];
    }
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      if (g < G) {
        const float y0 = conv_silu_hist(w0, h0, xa[g]);
        if (t < kD) {
          qn_s[g][t] = y0;
          v_s[g][t] = conv_silu_hist(w1, h1, xv[g]);
        } else {
          kn_s[g][t - kD] = y0;
        }
        h0[0] = h0[1];
        h0[1] = h0[2];
        h0[2] = xa[g];
        h1[0] = h1[1];
        h1[1] = h1[2];
        h1[2] = xv[g];
      }
    }
    __syncthreads();

    // 2. L2 norms, k.q and gates; wave w takes tokens w, w + 4, ...  The
    // normalised q and k replace the raw ones (each lane rewrites what it read).
    for (int g = wave; g < G; g += kWaves) {
      const float q0 = qn_s[g][lane], q1 = qn_s[g][lane + 64];
      const float k0 = kn_s[g][lane], k1 = kn_s[g][lane + 64];
      const float sq = wave_total(q0 * q0 + q1 * q1);
      const float sk = wave_total(k0 * k0 + k1 * k1);
      const float sqk = wave_total(q0 * k0 + q1 * k1);
      const float iq = (1.f / sqrtf(sq + kL2Eps)) * 0.08838834764831845f;  // 1/sqrt(128)
      const float ik = 1.f / sqrtf(sk + kL2Eps);
      const float kq = sqk * iq * ik;
      const float za = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ra), g)) + dtb;
      const float zb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rb), g));
      const float softplus = fmaxf(za, 0.f) + log1pf(expf(-fabsf(za)));
      const float alpha = expf(-expf(a_log) * softplus);
      const float eb = expf(-fabsf(zb));
      const float beta = zb >= 0.f ? 1.f / (1.f + eb) : eb / (1.f + eb);
      qn_s[g][lane] = q0 * iq;
      qn_s[g][lane + 64] = q1 * iq;
      kn_s[g][lane] = k0 * ik;
      kn_s[g][lane + 64] = k1 * ik;
      if (lane == 0) {
        al_s[g] = alpha;
        be_s[g] = beta;
        kq_s[g] = kq;
      }
    }
    __syncthreads();

    // 3. the recurrence over the group's tokens
    for (int g = 0; g < G; ++g) {
      const size_t tok = tok0 + g;
      float kr[kRows];
      float pk[8], pq[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pk[j] = pq[j] = 0.f;
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int row = rg + kRG * r;
        kr[r] = kn_s[g][row];
        const float qr = qn_s[g][row];
        if constexpr (kF32) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            pk[j] = fmaf(sf[r][j], kr[r], pk[j]);
            pq[j] = fmaf(sf[r][j], qr, pq[j]);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            pk[2 * k] = fma_f16<false>(kr[r], sw[r][k], pk[2 * k]);
            pk[2 * k + 1] = fma_f16<true>(kr[r], sw[r][k], pk[2 * k + 1]);
            pq[2 * k] = fma_f16<false>(qr, sw[r][k], pq[2 * k]);
            pq[2 * k + 1] = fma_f16<true>(qr, sw[r][k], pq[2 * k + 1]);
          }
        }
      }
      column_sums<kChunks, kCW>(pk, pq, red[wave], lane);
      __syncthreads();

      // u and the output, one column per thread
      if (t < kCW) {
        const float alpha = al_s[g], beta = be_s[g], kq = kq_s[g];
        float tk = 0.f, tq = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          tk += red[w][0][t];
          tq += red[w][1][t];
        }
        const int cc = slice * kCW + t;
        const float u = beta * (v_s[g][cc] - alpha * tk);
        const float o = fmaf(alpha, tq, u * kq);
        u_s[t] = u;
        pr.o[(tok * kVH + h) * kD + cc] = static_cast<uint16_t>(rma::f32_to_bf16(o));
      }
      __syncthreads();

      const float alpha = al_s[g];
      float u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) u[j] = u_s[8 * c + j];
      // the new elements, rounded as stored (the next step reads them back)
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        if constexpr (kF32) {
#pragma unroll
          for (int j = 0; j < 8; ++j) sf[r][j] = fmaf(alpha, sf[r][j], kr[r] * u[j]);
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            sw[r][k] = pack_f16x2(fma_f16<false>(alpha, sw[r][k], kr[r] * u[2 * k]),
                                  fma_f16<true>(alpha, sw[r][k], kr[r] * u[2 * k + 1]));
        }
      }
    }
  }

#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const size_t e = head + static_cast<size_t>(rg + kRG * i) * kD + col;
    if constexpr (kF32) {
      f32x4_t lo, hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo[j] = sf[i][j];
        hi[j] = sf[i][4 + j];
      }
      f32x4_t *dst = reinterpret_cast<f32x4_t *>(static_cast<float *>(pr.S) + e);
      __builtin_nontemporal_store(lo, dst);
      __builtin_nontemporal_store(hi, dst + 1);
    } else {
      const u32x4 w = {sw[i][0], sw[i][1], sw[i][2], sw[i][3]};
      __builtin_nontemporal_store(__builtin_bit_cast(f32x4_t, w),
                                  reinterpret_cast<f32x4_t *>(static_cast<_Float16 *>(pr.S) + e));
    }
  }
}

// The ring after the chunk: the inputs of its last min(T, 4) tokens, each in slot
// (its position) mod 4; the other slots keep what they held.  One workgroup per
// (sequence, slot); 256 threads copy the 8192 channels in 16-byte pieces.
__global__ __launch_bounds__(256) void gdn_prefill_ring_kernel(PrefillParams pr) {
  const int b = blockIdx.x / kConv;
  const int slot = blockIdx.x % kConv;
  const int T = pr.n_tokens;
  const int p0 = pr.pos[b];
  // the last token of the chunk that lands in this slot, if any
  const int last = p0 + T - 1;
  const int d = (last - slot) & 3;  // tokens back from the last one
  if (d >= T) return;
  const int i = T - 1 - d;
  const uint4 *src = reinterpret_cast<const uint4 *>(pr.x + (static_cast<size_t>(b) * T + i) * kCD);
  uint4 *dst = reinterpret_cast<uint4 *>(const_cast<uint16_t *>(pr.conv) +
                                         (static_cast<size_t>(b) * kConv + slot) * kCD);
  for (int e = threadIdx.x; e < kCD / 8; e += 256) dst[e] = src[e];
}

template <bool kF32, int kCW>
static void launch(const Params &pr, int batch, hipStream_t s) {
  hipLaunchKernelGGL((gdn_decode_kernel<kF32, kCW>), dim3(batch * kVH * (kD / kCW)),
                     dim3(kThreads), 0, s, pr);
}

}  // namespace gdn

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

extern "C" size_t gdn_layer_state_bytes(int32_t batch, int32_t state_dtype) {
  if (batch <= 0 || (state_dtype != GDN_STATE_F16 && state_dtype != GDN_STATE_F32)) return 0;
  const size_t eb = state_dtype == GDN_STATE_F32 ? 4 : 2;
  return static_cast<size_t>(batch) *
         (static_cast<size_t>(GDN_V_HEADS) * GDN_HEAD_DIM * GDN_HEAD_DIM * eb +
          static_cast<size_t>(GDN_CONV) * GDN_CONV_DIM * 2);
}

extern "C" rma_status gdn_decode_step(const gdn_layer_state *st, int32_t batch, int32_t state_dtype,
                                      const uint16_t *x, const float *a, const float *b,
                                      const int32_t *pos, const gdn_params *prm, uint16_t *o,
                                      void *stream) {
  if (!st || !prm || !x || !a || !b || !pos || !o) return RMA_E_ARG;
  if (!st->S || !st->conv || !prm->conv_w || !prm->a_log || !prm->dt_bias) return RMA_E_ARG;
  if (batch <= 0 || batch > RMA_MAX_BATCH) return RMA_E_ARG;
  if (state_dtype != GDN_STATE_F16 && state_dtype != GDN_STATE_F32) return RMA_E_ARG;
  const void *al[] = {st->S, st->conv, x, o, prm->conv_w};
  for (const void *p : al)
    if (!aligned16(p)) return RMA_E_ALIGN;
  gdn::Params pr;
  pr.S = st->S;
  pr.conv = st->conv;
  pr.x = x;
  pr.a = a;
  pr.b = b;
  pr.pos = pos;
  pr.conv_w = prm->conv_w;
  pr.a_log = prm->a_log;
  pr.dt_bias = prm->dt_bias;
  pr.o = o;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Below 16 sequences a head is split over 4 column slices of 32 so that the
  // launch still has 128+ workgroups.
  const bool wide = batch >= 16;
  if (state_dtype == GDN_STATE_F32) {
    if (wide)
      gdn::launch<true, RMA_GDN_WIDE_COLS>(pr, batch, s);
    else
      gdn::launch<true, 32>(pr, batch, s);
  } else {
    if (wide)
      gdn::launch<false, RMA_GDN_WIDE_COLS>(pr, batch, s);
    else
      gdn::launch<false, 32>(pr, batch, s);
  }
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  return RMA_OK;
}

extern "C" rma_status gdn_prefill(const gdn_layer_state *st, int32_t batch, int32_t n_tokens,
                                  int32_t state_dtype, const uint16_t *x, const float *a,
                                  const float *b, const int32_t *pos, const gdn_params *prm,
                                  uint16_t *o, void *stream) {
  if (!st || !prm || !x || !a || !b || !pos || !o) return RMA_E_ARG;
  if (!st->S || !st->conv || !prm->conv_w || !prm->a_log || !prm->dt_bias) return RMA_E_ARG;
  if (batch <= 0 || batch > RMA_MAX_BATCH) return RMA_E_ARG;
  if (n_tokens <= 0 || n_tokens > GDN_MAX_PREFILL) return RMA_E_ARG;
  if (state_dtype != GDN_STATE_F16 && state_dtype != GDN_STATE_F32) return RMA_E_ARG;
  const void *al[] = {st->S, st->conv, x, o, prm->conv_w};
  for (const void *p : al)
    if (!aligned16(p)) return RMA_E_ALIGN;
  gdn::PrefillParams pr;
  pr.S = st->S;
  pr.conv = st->conv;
  pr.x = x;
  pr.a = a;
  pr.b = b;
  pr.pos = pos;
  pr.conv_w = prm->conv_w;
  pr.a_log = prm->a_log;
  pr.dt_bias = prm->dt_bias;
  pr.o = o;
  pr.n_tokens = n_tokens;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the same column slices as the decode step at this batch (and so the same
  // arithmetic per token)
  const bool wide = batch >= 16;
  const unsigned per_head = wide ? gdn::kD / RMA_GDN_WIDE_COLS : gdn::kD / 32;
  const dim3 grid(static_cast<unsigned>(batch) * gdn::kVH * per_head);
  if (state_dtype == GDN_STATE_F32) {
    if (wide)
      hipLaunchKernelGGL((gdn::gdn_prefill_kernel<true, RMA_GDN_WIDE_COLS>), grid,
                         dim3(gdn::kThreads), 0, s, pr);
    else
      hipLaunchKernelGGL((gdn::gdn_prefill_kernel<true, 32>), grid, dim3(gdn::kThreads), 0, s, pr);
  } else {
    if (wide)
      hipLaunchKernelGGL((gdn::gdn_prefill_kernel<false, RMA_GDN_WIDE_COLS>), grid,
                         dim3(gdn::kThreads), 0, s, pr);
    else
      hipLaunchKernelGGL((gdn::gdn_prefill_kernel<false, 32>), grid, dim3(gdn::kThreads), 0, s, pr);
  }
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  hipLaunchKernelGGL(gdn::gdn_prefill_ring_kernel, dim3(static_cast<unsigned>(batch) * GDN_CONV),
                     dim3(256), 0, s, pr);
  if (hipPeekAtLastError() != hipSuccess) return (void)hipGetLastError(), RMA_E_HIP;
  return RMA_OK;
}
