// Rotate+quant of short rows (d = 32 .. 256, a power of two): four lanes of
// a wave own one row.  Used for the per-head K/V groups and for short
// activation rows.
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary), section 3.4 Stage 1d (head-wise Hadamard on keys after RoPE) and
// Stage 2c (one quantisation group per head vector); "QuaRot Guide",
// section 3 of "The Architecture" (fast Walsh-Hadamard transform: d log d
// additions and subtractions, no multiplies).
//
// Layout.  Lane q (0..3) of a quad owns the 16-byte chunks c = q + 4j of the
// row, j = 0..D/32-1, so element e = 8q + 32j + i (i = 0..7) sits in register
// r = 8j + i.  Element bits 0-2 and 5.. are register bits (butterflies
// inside a lane); element bits 3 and 4 are lane bits 0 and 1 of the quad
// (butterflies through DPP quad permutations).  Loads are 16 contiguous bytes
// per lane, four lanes cover 64 contiguous bytes; each chunk's eight codes
// pack into one 32-bit word.
#pragma once

#include "quant_common.h"

namespace quarot {

// The two quad butterfly stages (partner lane ^ 1, then ^ 2) on E registers,
// each as v + partner * c in one v_fmac_f32 with DPP, c = +1 on the low lane
// and -1 on the high lane.  A high lane ends with b - a instead of a - b, so
// afterwards every value of lane q carries the sign (-1)^(q0 + q1), which the
// quantisers fold into their scale.  DPP needs two wait states after a VALU
// write of its source: stage 1 reads only what stage 0's blocks
// wrote at least E - 4 instructions earlier, and the last block closes with
// s_nop 1.  (Every stage-0 block opens with s_nop 1: the compiler may
// schedule the producer of any register right before it.)
template <int E>
__device__ __forceinline__ void quad_butterflies(float (&v)[E], float c0, float c1) {
  static_assert(E % 4 == 0 && E >= 8, "blocks of four registers");
#define QR_QUAD_DPP(LEAD, CTRL, C, TRAIL)                                                    \
  asm volatile(LEAD                                                                          \
               "v_fmac_f32_dpp %0, %0, %4 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               "v_fmac_f32_dpp %1, %1, %4 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               "v_fmac_f32_dpp %2, %2, %4 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               "v_fmac_f32_dpp %3, %3, %4 " CTRL " row_mask:0xf bank_mask:0xf" TRAIL      \
               : "+v"(v[r]), "+v"(v[r + 1]), "+v"(v[r + 2]), "+v"(v[r + 3])              \
               : "v"(C))
#pragma unroll
  for (int r = 0; r < E; r += 4) {
    QR_QUAD_DPP("s_nop 1\n", "quad_perm:[1,0,3,2]", c0, "");
  }
#pragma unroll
  for (int r = 0; r < E; r += 4) {
    if (r + 4 < E) QR_QUAD_DPP("", "quad_perm:[2,3,0,1]", c1, "");
    else QR_QUAD_DPP("", "quad_perm:[2,3,0,1]", c1, "\ns_nop 1");
  }
#undef QR_QUAD_DPP
}

template <int LB>
__device__ __forceinline__ float quad_max(float v) {
  constexpr int ctrl = (LB == 0) ? 0xB1 : 0x4E;
  const float p = __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF, 0xF, true));
  return fmaxf(v, p);
}

// XOR masks that flip the fp16 sign bits of this lane's elements (chunk
// c = q + 4j holds elements 8c .. 8c + 7); all loads issue before any use.
template <int NC>
__device__ __forceinline__ void load_sign_masks(const int8_t* sg, int q, uint4 (&mask)[NC]) {
  if (!sg) {
#pragma unroll
    for (int j = 0; j < NC; ++j) mask[j] = make_uint4(0, 0, 0, 0);
    return;
  }
  uint32_t w[NC][2];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    __builtin_memcpy(&w[j][0], sg + 8 * (q + 4 * j), 4);
    __builtin_memcpy(&w[j][1], sg + 8 * (q + 4 * j) + 4, 4);
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) mask[j] = sign_masks8(w[j][0], w[j][1]);
}

// The raw fp16 chunks of one row held by a quad.  The caller passes a valid
// row address even for an inactive quad (whose values are then unused), so
// the loads carry no condition.
template <int D>
__device__ __forceinline__ void quad_load(const __half* __restrict__ src, int q,
                                          uint4 (&raw)[D / 32]) {
#pragma unroll
  for (int j = 0; j < D / 32; ++j) raw[j] = *reinterpret_cast<const uint4*>(src + 8 * (q + 4 * j));
}

// 1 / sqrt(D) for the supported head dimensions.
template <int D>
__device__ __forceinline__ constexpr float quad_norm() {
  return 1.0f / (D == 32 ? 5.656854249492380f
                 : D == 64 ? 8.0f
                 : D == 128 ? 11.313708498984761f
                            : 16.0f);
}

// The unnormalised transform of one row held by a quad: sign flip, then the
// Sylvester butterflies (register bits, then the two lane bits by DPP).
// x~ = quad_sigma(q) * v / sqrt(D).  An inactive quad transforms zeros.
template <int D>
__device__ __forceinline__ void quad_transform(const uint4 (&raw)[D / 32],
                                               const uint4 (&mask)[D / 32], int q, bool active,
                                               float (&v)[D / 4]) {
  constexpr int NC = D / 32;  // chunks per lane
  constexpr int E = 8 * NC;   // elements per lane
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    uint4 r = raw[j];
    if (!active) r = make_uint4(0, 0, 0, 0);
    r.x ^= mask[j].x;
    r.y ^= mask[j].y;
    r.z ^= mask[j].z;
    r.w ^= mask[j].w;
    unpack_half8(r, &v[8 * j]);
  }
  // register-bit butterflies
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int r = 0; r < E; ++r) {
      if ((r & h) == 0) {
        const float a = v[r], b = v[r + h];
        v[r] = a + b;
        v[r + h] = a - b;
      }
    }
  }
  // lane-bit butterflies (element bits 3 and 4); every lane of the wave takes
  // part so the DPP sources are always defined
  quad_butterflies<E>(v, (q & 1) ? -1.0f : 1.0f, (q & 2) ? -1.0f : 1.0f);
}

// Sign that quad_transform leaves on lane q's values.
__device__ __forceinline__ float quad_sigma(int q) {
  return (((q ^ (q >> 1)) & 1) != 0) ? -1.0f : 1.0f;
}

// Rotate+quant (symmetric) of one row held by a quad, its raw chunks already
// loaded.  qrow: code row (D/2 bytes); scale: where the fp16 scale goes;
// xrot: optional fp32 row.

template <int D, bool CLAMP>
__device__ __forceinline__ void quad_row(const uint4 (&raw)[D / 32], uint8_t* __restrict__ qrow,
                                         __half* __restrict__ scale, float* __restrict__ xrot,
                                         const uint4 (&mask)[D / 32], int q, float clip_ratio,
                                         bool active) {
  constexpr int NC = D / 32;
  constexpr int E = 8 * NC;
  constexpr float kNorm = quad_norm<D>();
  float v[E];
  quad_transform<D>(raw, mask, q, active, v);
  // the transform is unnormalised: max|x~| = max|v| / sqrt(D)
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < E; ++r) amax = fmaxf(amax, fabsf(v[r]));
  amax = quad_max<0>(amax);
  amax = quad_max<1>(amax);
  const __half s16 = row_scale_fp16(amax * kNorm, clip_ratio);
  if (!active) return;
  const float sigma = quad_sigma(q);
  const float kq = inv_scale(s16) * kNorm * sigma;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    float t8[8];
    if (CLAMP) {
#pragma unroll
      for (int i = 0; i < 8; ++i) t8[i] = magic_code<true>(v[8 * j + i], kq);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) t8[i] = magic_code<false>(v[8 * j + i], kq);
    }
    *reinterpret_cast<uint32_t*>(qrow + 4 * (q + 4 * j)) = pack8_magic(t8);
  }
  if (q == 0) *scale = s16;
  if (xrot) {
    const float xn = kNorm * sigma;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      float4* dst = reinterpret_cast<float4*>(xrot + 8 * (q + 4 * j));
      dst[0] = make_float4(v[8 * j + 0] * xn, v[8 * j + 1] * xn, v[8 * j + 2] * xn,
                           v[8 * j + 3] * xn);
      dst[1] = make_float4(v[8 * j + 4] * xn, v[8 * j + 5] * xn, v[8 * j + 6] * xn,
                           v[8 * j + 7] * xn);
    }
  }
}

template <int LB>
__device__ __forceinline__ float quad_min(float v) {
  constexpr int ctrl = (LB == 0) ? 0xB1 : 0x4E;
  const float p = __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF, 0xF, true));
  return fminf(v, p);
}

// Rotate+quant (asymmetric, one zero point per group) of one row held by a
// quad.  "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs"
// (paper-graph-ui summary), section 3.4 Stage 2c: the range is the clipped
// min and max of the group, S = fp16(max(range, 1e-5) / 15), the zero point
// z = rint(-alpha_min / S) kept within +-1024 (stored as fp16, exact), and
// the uint4 code q = clamp(rint(x / S) + z, 0, 15); element 2k in the low
// nibble of byte k.  xrot: optional fp32 row receiving x~.
template <int D>
__device__ __forceinline__ void quad_row_asym(const uint4 (&raw)[D / 32],
                                              uint8_t* __restrict__ qrow,
                                              __half* __restrict__ scale,
                                              __half* __restrict__ zero,
                                              float* __restrict__ xrot,
                                              const uint4 (&mask)[D / 32], int q,
                                              float clip_ratio, bool active) {
  constexpr int NC = D / 32;
  constexpr int E = 8 * NC;
  constexpr float kNorm = quad_norm<D>();
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: integers in the low mantissa bits
  float v[E];
  quad_transform<D>(raw, mask, q, active, v);
  float vmin = v[0], vmax = v[0];
#pragma unroll
  for (int r = 1; r < E; ++r) {
    vmin = fminf(vmin, v[r]);
    vmax = fmaxf(vmax, v[r]);
  }
  // the lane's values are sigma * x~ * sqrt(D): a negative sigma swaps and
  // negates the extremes
  const float sigma = quad_sigma(q);
  if (sigma < 0.0f) {
    const float t = vmin;
    vmin = -vmax;
    vmax = -t;
  }
  vmin = quad_min<1>(quad_min<0>(vmin));
  vmax = quad_max<1>(quad_max<0>(vmax));
  // scaling by the positive 1 / sqrt(D) keeps the extremes
  const float amin = clip_ratio * (vmin * kNorm);
  const float amax = clip_ratio * (vmax * kNorm);
  const float range = fmaxf(amax - amin, 1e-5f);
  // range / 15 and x / S as products with reciprocals (v_rcp_f32, about one
  // ulp): the three fp32 divisions were a fifth of the group's VALU work; a
  // scale, zero point or code can then differ from the exact division's
  // where the quotient sits within an ulp or two of a rounding boundary
  const __half s16 = __float2half_rn(range * (1.0f / 15.0f));
  const float sf = __half2float(s16);
  const float rs = __builtin_amdgcn_rcpf(sf);
  const float z = fminf(fmaxf(__builtin_rintf(-amin * rs), -1024.0f), 1024.0f);
  if (!active) return;
  const float kq = rs * kNorm * sigma;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    float t8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // rint(x / S) + M, then + z (both integers, exact), clamped to [M, M + 15]
      const float t = fmaf(v[8 * j + i], kq, kMagic) + z;
      t8[i] = fminf(fmaxf(t, kMagic), kMagic + 15.0f);
    }
    const uint32_t ev = gather_byte0(t8[0], t8[2], t8[4], t8[6]);
    const uint32_t od = gather_byte0(t8[1], t8[3], t8[5], t8[7]);
    *reinterpret_cast<uint32_t*>(qrow + 4 * (q + 4 * j)) = (od << 4) | ev;
  }
  if (q == 0) {
    *scale = s16;
    *zero = __float2half_rn(z);
  }
  if (xrot) {
    const float xn = kNorm * sigma;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      float4* dst = reinterpret_cast<float4*>(xrot + 8 * (q + 4 * j));
      dst[0] = make_float4(v[8 * j + 0] * xn, v[8 * j + 1] * xn, v[8 * j + 2] * xn,
                           v[8 * j + 3] * xn);
      dst[1] = make_float4(v[8 * j + 4] * xn, v[8 * j + 5] * xn, v[8 * j + 6] * xn,
                           v[8 * j + 7] * xn);
    }
  }
}

}  // namespace quarot
