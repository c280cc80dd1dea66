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

namespace quarot {

// Round to nearest integer by the float "magic number" addition: for
// |v| < 2^22, fma(y, k, 1.5 * 2^23 + 8) rounds y * k to the nearest integer
// q (ties to even, the current rounding mode) and leaves q + 8 in the low
// bits of the result, so byte 0 of its bit pattern is q + 8 in [0, 15]
// whenever q is in [-8, 7].
constexpr float kMagic8 = 12582912.0f + 8.0f;

// q + 8 in byte 0 of the returned float's bits; CLAMP limits q to [-8, 7].
template <bool CLAMP>
__device__ __forceinline__ float magic_code(float y, float k) {
  float t = fmaf(y, k, kMagic8);
  if (CLAMP) t = fminf(fmaxf(t, kMagic8 - 8.0f), kMagic8 + 7.0f);
  return t;
}

// Byte 0 of four words, gathered into one word (a in byte 0 ... d in byte 3).
__device__ __forceinline__ uint32_t gather_byte0(float a, float b, float c, float d) {
  const uint32_t ab = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b),
                                            __builtin_bit_cast(uint32_t, a), 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, d),
                                            __builtin_bit_cast(uint32_t, c), 0x0c0c0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Eight magic_code results (element i in t[i]) -> one word, code i in nibble i
// as 4-bit two's complement: evens fill the low nibbles of each byte, odds
// the high nibbles, and xor 8 turns the q + 8 offset into two's complement.
__device__ __forceinline__ uint32_t pack8_magic(const float* t) {
  const uint32_t ev = gather_byte0(t[0], t[2], t[4], t[6]);
  const uint32_t od = gather_byte0(t[1], t[3], t[5], t[7]);
  return ((od << 4) | ev) ^ 0x88888888u;
}

// XOR masks flipping the fp16 sign bits of 8 consecutive elements whose
// int8 signs (+1 / -1, sign bit = bit 7) are the bytes of w0 (elements 0-3)
// and w1 (elements 4-7).
// Each mask word is one byte permute (sign bytes into bytes 1 and 3) and an AND.
__device__ __forceinline__ uint4 sign_masks8(uint32_t w0, uint32_t w1) {
  uint4 m;
  m.x = __builtin_amdgcn_perm(w0, w0, 0x010c000cu) & 0x80008000u;
  m.y = __builtin_amdgcn_perm(w0, w0, 0x030c020cu) & 0x80008000u;
  m.z = __builtin_amdgcn_perm(w1, w1, 0x010c000cu) & 0x80008000u;
  m.w = __builtin_amdgcn_perm(w1, w1, 0x030c020cu) & 0x80008000u;
  return m;
}

}  // namespace quarot
