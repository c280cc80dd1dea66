// Rotate+quant of rows of d = 4096 (a power of two): one wave owns one row.
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary), section 3.4 Stage 1a (R = H diag(s)) and Stage 2b (per-token
// symmetric INT4); "QuaRot Guide", section 3 of "The Architecture" (FWHT by
// additions and subtractions only).
//
// The 12 butterfly stages over the element index e (bits e0..e11) are split
// into two phases around one exchange through LDS:
//   phase 1  lane l loads chunk j (j = 0..7) = elements 512 j + 8 l + i, so
//            e0-e2 (i) and e9-e11 (j) are register bits and e3-e8 lane bits.
//            Butterflies on the six register bits in registers, on e3 and e4
//            through DPP quad permutations and on e6 through DPP row_ror:8.
//   exchange the row (fp32, 16 KiB) goes through the wave's own LDS slice.
//   phase 2  lane l' holds e3, e4, e6, e9, e10, e11 as lane bits and e0-e2,
//            e5, e7, e8 as register bits; butterflies on e5, e7, e8.
// Phase 2 keeps eight consecutive elements per register group, so the codes
// of a group pack into one 32-bit word.  The absolute maximum is a wave
// reduction; the codes come from one fma with the float magic number.
#pragma once

#include "quant_common.h"

namespace quarot {

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Low lane keeps a + b, high lane keeps a - b (sgn = +1 low, -1 high).
template <int CTRL>
__device__ __forceinline__ float dpp_butterfly(float v, float sgn) {
  return fmaf(v, sgn, dpp_mov<CTRL>(v));
}

constexpr int kDppQuadX1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadX2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowRor8 = 0x128; // row_ror:8 (partner lane ^ 8 inside 16)

__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_mov<kDppQuadX1>(v));
  v = fmaxf(v, dpp_mov<kDppQuadX2>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_mov<0x140>(v));  // row_mirror
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// Physical float4 slot of logical float4 chunk c (= element / 4) in a wave's
// 4096-float LDS slice: flips bit 0 by e5 ^ e6 so both access patterns
// spread over the banks.
__device__ __forceinline__ int x4096_slot(int c) { return c ^ (((c >> 3) ^ (c >> 4)) & 1); }

constexpr int kWaveRowsBlock = 256;  // 4 waves, one row each

template <bool CLAMP>
__global__ __launch_bounds__(kWaveRowsBlock) void had_quant_4096(
    const __half* __restrict__ x, int64_t rows, int64_t ld_x, const int8_t* __restrict__ signs,
    float clip_ratio, uint8_t* __restrict__ q_out, int64_t ld_q, __half* __restrict__ scale_out,
    float* __restrict__ x_rot) {
  __shared__ float4 lds[kWaveRowsBlock / 64][1024];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float4* slice = lds[wave];

  // sign masks for this lane's phase-1 elements (flip fp16 sign bits)
  uint32_t mask[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t mk = 0;
      if (signs) {
        const int e = 512 * j + 8 * lane + 2 * p;
        mk = (signs[e] < 0 ? 0x8000u : 0u) | (signs[e + 1] < 0 ? 0x80000000u : 0u);
      }
      mask[j][p] = mk;
    }
  const float s_q1 = (lane & 1) ? -1.0f : 1.0f;
  const float s_q2 = (lane & 2) ? -1.0f : 1.0f;
  const float s_r8 = (lane & 8) ? -1.0f : 1.0f;
  // phase-2 element base of this lane (i = 0, k = 0)
  const int e2base = 8 * (lane & 1) + 16 * ((lane >> 1) & 1) + 64 * ((lane >> 2) & 1) +
                     512 * (lane >> 3);

  const int64_t wstride = int64_t(gridDim.x) * (kWaveRowsBlock / 64);
  int64_t row = int64_t(blockIdx.x) * (kWaveRowsBlock / 64) + wave;
  uint4 raw[8];
  if (row < rows) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      raw[j] = *reinterpret_cast<const uint4*>(x + row * ld_x + 512 * j + 8 * lane);
  }
  for (; row < rows; row += wstride) {
    float v[64];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint4 r = raw[j];
      r.x ^= mask[j][0];
      r.y ^= mask[j][1];
      r.z ^= mask[j][2];
      r.w ^= mask[j][3];
      unpack_half8(r, &v[8 * j]);
    }
    // prefetch the next row of this wave
    const int64_t nrow = row + wstride;
    if (nrow < rows) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        raw[j] = *reinterpret_cast<const uint4*>(x + nrow * ld_x + 512 * j + 8 * lane);
    }
    // phase 1: register bits (e0-e2 = r bits 0-2, e9-e11 = r bits 3-5)
#pragma unroll
    for (int h = 1; h < 64; h <<= 1)
#pragma unroll
      for (int r = 0; r < 64; ++r)
        if ((r & h) == 0) {
          const float a = v[r], b = v[r + h];
          v[r] = a + b;
          v[r + h] = a - b;
        }
    // phase 1: lane bits through DPP (e3, e4, e6)
#pragma unroll
    for (int r = 0; r < 64; ++r) v[r] = dpp_butterfly<kDppQuadX1>(v[r], s_q1);
#pragma unroll
    for (int r = 0; r < 64; ++r) v[r] = dpp_butterfly<kDppQuadX2>(v[r], s_q2);
#pragma unroll
    for (int r = 0; r < 64; ++r) v[r] = dpp_butterfly<kDppRowRor8>(v[r], s_r8);
    // exchange: element e lives in float4 slot x4096_slot(e / 4)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = (512 * j + 8 * lane + 4 * h) >> 2;
        slice[x4096_slot(c)] = make_float4(v[8 * j + 4 * h], v[8 * j + 4 * h + 1],
                                           v[8 * j + 4 * h + 2], v[8 * j + 4 * h + 3]);
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
    // phase 2 registers: r' = 8 k + i, k bits = (e5, e7, e8)
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = e2base + 32 * (k & 1) + 128 * ((k >> 1) & 1) + 256 * (k >> 2) + 4 * h;
        const float4 f = slice[x4096_slot(e >> 2)];
        v[8 * k + 4 * h] = f.x;
        v[8 * k + 4 * h + 1] = f.y;
        v[8 * k + 4 * h + 2] = f.z;
        v[8 * k + 4 * h + 3] = f.w;
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int h = 8; h < 64; h <<= 1)
#pragma unroll
      for (int r = 0; r < 64; ++r)
        if ((r & h) == 0) {
          const float a = v[r], b = v[r + h];
          v[r] = a + b;
          v[r + h] = a - b;
        }
    // scale: the FWHT is unnormalised; 1/sqrt(4096) = 1/64 is exact
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 64; ++r) amax = fmaxf(amax, fabsf(v[r]));
    amax = wave_max_dpp(amax) * (1.0f / 64.0f);
    const __half s16 = row_scale_fp16(amax, clip_ratio);
    const float k = inv_scale(s16) * (1.0f / 64.0f);
    uint8_t* qrow = q_out + row * ld_q;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = magic_code<CLAMP>(v[8 * kk + i], k);
      const int e0 = e2base + 32 * (kk & 1) + 128 * ((kk >> 1) & 1) + 256 * (kk >> 2);
      *reinterpret_cast<uint32_t*>(qrow + (e0 >> 1)) = pack8_magic(t);
    }
    if (lane == 0) scale_out[row] = s16;
    if (x_rot) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int e0 = e2base + 32 * (kk & 1) + 128 * ((kk >> 1) & 1) + 256 * (kk >> 2);
        float4* dst = reinterpret_cast<float4*>(x_rot + row * 4096 + e0);
        const float c = 1.0f / 64.0f;
        dst[0] = make_float4(v[8 * kk] * c, v[8 * kk + 1] * c, v[8 * kk + 2] * c, v[8 * kk + 3] * c);
        dst[1] = make_float4(v[8 * kk + 4] * c, v[8 * kk + 5] * c, v[8 * kk + 6] * c,
                             v[8 * kk + 7] * c);
      }
    }
  }
}

}  // namespace quarot
