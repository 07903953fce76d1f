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

// Rotary angle of pair i at position p, computed in double so that positions
// up to 2^18 keep full FP32 accuracy in cos/sin.
__device__ __forceinline__ void rope_cos_sin(int i, int p, float base, float &c, float &s) {
  double theta = pow(static_cast<double>(base), -2.0 * static_cast<double>(i) / kRope);
  double phi = static_cast<double>(p) * theta;
  double sd, cd;
  sincos(phi, &sd, &cd);
  c = static_cast<float>(cd);
  s = static_cast<float>(sd);
}

// RMS-normalise one 256-wide head held by a wave (lane l holds dims 4l..4l+3),
// multiply by the gain, then rotate dims 0..63 at position p (pairs i, i+32).
// x is updated in place.  Lanes 0..7 hold the first half of the rotated dims
// and lanes 8..15 their partners.
__device__ __forceinline__ void norm_rope_head(float x[4], const float *gamma, float eps, int p,
                                               float base, int lane) {
  float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss * (1.0f / kDim) + eps);
  const float4 gm = *reinterpret_cast<const float4 *>(gamma + 4 * lane);
  x[0] = x[0] * inv * gm.x;
  x[1] = x[1] * inv * gm.y;
  x[2] = x[2] * inv * gm.z;
  x[3] = x[3] * inv * gm.w;
  float partner[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) partner[e] = __shfl_xor(x[e], 8, 64);
  if (lane < 16) {
    const bool first = lane < 8;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * (lane & 7) + e;
      float c, s;
      rope_cos_sin(i, p, base, c, s);
      // first half:  y_i      = x_i c - x_{i+32} s
      // second half: y_{i+32} = x_{i+32} c + x_i s
      x[e] = first ? (x[e] * c - partner[e] * s) : (x[e] * c + partner[e] * s);
    }
  }
}

}  // namespace rma
