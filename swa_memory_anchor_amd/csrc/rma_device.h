// Device helpers shared by the RMA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rma.h"

namespace rma {

constexpr int kHeads = RMA_Q_HEADS;
constexpr int kGroups = RMA_KV_GROUPS;
constexpr int kDim = RMA_HEAD_DIM;
constexpr int kRope = RMA_ROPE_DIM;
constexpr int kWindow = RMA_WINDOW;
constexpr int kBank = RMA_BANK;
constexpr int kBlock = RMA_BLOCK;
constexpr int kHidden = RMA_HIDDEN;
constexpr int kMid = RMA_SCORER_MID;
constexpr int kHeadsPerGroup = kHeads / kGroups;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bf16 bits, round to nearest even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Rotary frequencies theta_i = base^(-2i/64) = r^i with r = base^(-1/32).  r is
// computed on the host in double precision; each lane forms r^i by binary
// powering in double (at most 9 multiplies, relative error below 1e-15).
inline double rope_ratio(float base) { return __builtin_pow(static_cast<double>(base), -2.0 / kRope); }

// (cos, sin) of pair i = lane % 32 at position p.  The angle p * theta_i is formed
// and reduced modulo 2*pi in double (Cody-Waite, two-term 2*pi), so positions up
// to 2^18 keep full accuracy.  The reduced angle r (|r| <= pi) is split into
// rf = fp32(r) and the remainder d = r - rf; sin and cos of rf are taken in FP32
// and corrected to first order in d (|d| <= 2^-22, so the second-order term is
// below FP32 resolution).
__device__ __forceinline__ void rope_cos_sin_theta(double theta, int p, float &c, float &s) {
  constexpr double kTwoPiHi = 6.283185307179586232;       // 2*pi rounded to double
  constexpr double kTwoPiLo = 2.4492935982947064e-16;      // 2*pi - kTwoPiHi
  constexpr double kInvTwoPi = 0.15915494309189534561;
  const double phi = static_cast<double>(p) * theta;
  const double k = rint(phi * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, phi);
  r = fma(-k, kTwoPiLo, r);
  const float rf = static_cast<float>(r);
  const float d = static_cast<float>(r - static_cast<double>(rf));
  const float s0 = sinf(rf), c0 = cosf(rf);
  s = fmaf(c0, d, s0);
  c = fmaf(-s0, d, c0);
}

__device__ __forceinline__ void rope_cos_sin(double ratio, int p, int lane, float &c, float &s) {
  int i = lane & (kRope / 2 - 1);
  double theta = 1.0, sq = ratio;
  while (i) {
    if (i & 1) theta *= sq;
    sq *= sq;
    i >>= 1;
  }
  rope_cos_sin_theta(theta, p, c, s);
}

// RMS-normalise one 256-wide head held by a wave (lane l holds dims 4l..4l+3),
// multiply by the gain, then rotate dims 0..63 at the position whose per-pair
// (cos, sin) lane i < 32 holds in (c, s) (pairs i, i+32).  Lanes 0..7 hold the
// first half of the rotated dims and lanes 8..15 their partners.
__device__ __forceinline__ void norm_rope_head(float x[4], const float *gamma, float eps, float c,
                                               float s, int lane) {
  float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss * (1.0f / kDim) + eps);
  const float4 gm = *reinterpret_cast<const float4 *>(gamma + 4 * lane);
  x[0] = x[0] * inv * gm.x;
  x[1] = x[1] * inv * gm.y;
  x[2] = x[2] * inv * gm.z;
  x[3] = x[3] * inv * gm.w;
  float partner[4], ce[4], se[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    partner[e] = __shfl_xor(x[e], 8, 64);
    ce[e] = __shfl(c, 4 * (lane & 7) + e, 64);
    se[e] = __shfl(s, 4 * (lane & 7) + e, 64);
  }
  if (lane < 16) {
    const bool first = lane < 8;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // first half:  y_i      = x_i c - x_{i+32} s
      // second half: y_{i+32} = x_{i+32} c + x_i s
      x[e] = first ? (x[e] * ce[e] - partner[e] * se[e]) : (x[e] * ce[e] + partner[e] * se[e]);
    }
  }
}

}  // namespace rma
