// Device helpers shared by the rotate+quant kernels: the per-token scale,
// the round-to-nearest INT4 code and nibble packing.
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary), section 3.4 Stage 2b: symmetric per-token scale
// s = clip * max|x| / 7; "QuaRot Guide", section 3 of "The Problem": codes are
// clip(round(x / S), -8, 7); its code floors the absolute maximum at 1e-5.
#pragma once

#include "common.h"

namespace quarot {

// fp16 scale from the row's absolute maximum (already normalised by 1/sqrt(d)).
__device__ __forceinline__ __half row_scale_fp16(float amax, float clip_ratio) {
  const float a = fmaxf(amax, 1e-5f);
  return __float2half_rn((clip_ratio * a) / 7.0f);
}

// 1 / S for the stored fp16 scale.
__device__ __forceinline__ float inv_scale(__half s) { return 1.0f / __half2float(s); }

// Round-to-nearest-even code of x * k, clamped to [-8, 7], as a 4-bit field.
__device__ __forceinline__ uint32_t int4_code(float x, float k) {
  float r = __builtin_rintf(x * k);
  r = fminf(fmaxf(r, -8.0f), 7.0f);
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xFu;
}

// Pack 8 consecutive codes (element i in nibble i) into one 32-bit word.
__device__ __forceinline__ uint32_t pack8(const float* v, float k) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= int4_code(v[i], k) << (4 * i);
  return w;
}

// fp16 x8 (one 16-byte load) -> fp32 x8.
__device__ __forceinline__ void unpack_half8(const uint4& raw, float* out) {
  const __half2* h = reinterpret_cast<const __half2*>(&raw);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float2 f = __half22float2(h[i]);
    out[2 * i] = f.x;
    out[2 * i + 1] = f.y;
  }
}

// Wave-wide max (64 lanes) of non-negative values.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace quarot
