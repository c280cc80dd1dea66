// Rotate+quant of rows of d = 4096 (a power of two): one wave owns one row.
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary), section 3.4 Stage 1a (R = H diag(s)), Stage 1b (online Hadamard
// in FP32) and Stage 2b (per-token symmetric INT4); "QuaRot Guide",
// section 3 of "The Architecture" (the fast transform).
//
// H_4096 = H_128 (x) H_32 as a Kronecker product over the element index
// bits: the H_32 factor over the five lowest bits is a dense 32 x 32
// contraction of the raw fp16 input and runs on the matrix cores; the
// remaining seven bits are butterflies (in registers, one DPP stage) around
// one exchange through LDS.  The absolute maximum is a wave reduction; the
// codes come from one fma with the float magic number.
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

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Physical float4 slot of logical float4 chunk c (= element / 4) in a wave's
// 4096-float LDS slice.  Bits 0-3 of the slot are XORed with bits 6, 4, 5, 7
// of c, so the sixteen lanes of an LDS cycle hit sixteen different 16-byte
// bank groups both when the MFMA layout writes and when phase 2 reads.
__device__ __forceinline__ int x4096_slot(int c) {
  return c ^ (((c >> 6) & 1) | (((c >> 4) & 1) << 1) | (((c >> 5) & 1) << 2) |
              (((c >> 7) & 1) << 3));
}

constexpr int kWaveRowsBlock = 256;  // 4 waves, one row each per iteration

// d = 4096, one wave per row.
//   phase 1  lane l = n + 16 g loads, for tile t = 0..7, elements
//            512 t + 32 n + 8 g + (0..7): the B operand of
//            v_mfma_f32_16x16x32_f16 (K = 8 g + j, N = n).  Two MFMAs with
//            the rows 0-15 and 16-31 of the Sylvester H_32 as A apply the
//            transform over element bits e0-e4 to the raw (sign-flipped)
//            fp16 input: products with +-1 are exact, sums are fp32.  The
//            output lands as elements 512 t + 32 n + 16 h + 4 g + (0..3).
//            Butterflies over e9-e11 (tile t) run in registers.
//   exchange through the wave's own LDS slice (fp32, 16 KiB).
//   phase 2  lane bits are e3, e4, e9, e8, e10, e11; register bits e0-e2,
//            e5, e6, e7.  Butterflies over e5-e7 in registers and over e8
//            through DPP row_ror:8.  Eight consecutive elements per
//            register group pack into one 32-bit word of codes.
template <bool CLAMP>
__global__ __launch_bounds__(kWaveRowsBlock, 2) void had_quant_4096(
    const __half* __restrict__ x, int64_t rows, int64_t ld_x, const int8_t* __restrict__ signs,
    float clip_ratio, uint8_t* __restrict__ q_out, int64_t ld_q, __half* __restrict__ scale_out,
    float* __restrict__ x_rot) {
  __shared__ float4 lds[kWaveRowsBlock / 64][1024];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float4* slice = lds[wave];
  const int n = lane & 15, g = lane >> 4;
  const int64_t wstride = int64_t(gridDim.x) * (kWaveRowsBlock / 64);
  int64_t row = int64_t(blockIdx.x) * (kWaveRowsBlock / 64) + wave;

  // issue the first row's loads before anything else
  uint4 raw[8];
  if (row < rows) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      raw[t] = *reinterpret_cast<const uint4*>(x + row * ld_x + 512 * t + 32 * n + 8 * g);
  }
  // sign masks of this lane's phase-1 elements (the same for every row)
  // (all eight loads are issued before the first use)
  uint4 mask[8];
  if (signs) {
    uint2 w[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
      w[t] = *reinterpret_cast<const uint2*>(signs + 512 * t + 32 * n + 8 * g);
#pragma unroll
    for (int t = 0; t < 8; ++t) mask[t] = sign_masks8(w[t].x, w[t].y);
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) mask[t] = make_uint4(0, 0, 0, 0);
  }
  // A operands: rows n and n + 16 of H_32, columns 8 g + j
  half8_t h_lo, h_hi;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = 8 * g + j;
    h_lo[j] = (__builtin_popcount(n & k) & 1) ? _Float16(-1.0f) : _Float16(1.0f);
    h_hi[j] = (__builtin_popcount((n + 16) & k) & 1) ? _Float16(-1.0f) : _Float16(1.0f);
  }
  const float s_r8 = (lane & 8) ? -1.0f : 1.0f;
  // phase-2 element base of this lane (e0-e2 = 0, e5-e7 = 0)
  const int e2base = 8 * (lane & 1) + 16 * ((lane >> 1) & 1) + 512 * ((lane >> 2) & 1) +
                     256 * ((lane >> 3) & 1) + 1024 * ((lane >> 4) & 1) + 2048 * (lane >> 5);

  for (; row < rows; row += wstride) {
    float v[64];
    // phase 1: H_32 over e0-e4 on the matrix cores
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint4 r = raw[t];
      r.x ^= mask[t].x;
      r.y ^= mask[t].y;
      r.z ^= mask[t].z;
      r.w ^= mask[t].w;
      const half8_t b = __builtin_bit_cast(half8_t, r);
      const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
      const float4_t d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(h_lo, b, zero, 0, 0, 0);
      const float4_t d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(h_hi, b, zero, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[8 * t + q] = d0[q];
        v[8 * t + 4 + q] = d1[q];
      }
    }
    // prefetch the next row of this wave
    const int64_t nrow = row + wstride;
    if (nrow < rows) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        raw[t] = *reinterpret_cast<const uint4*>(x + nrow * ld_x + 512 * t + 32 * n + 8 * g);
    }
    // phase 1: e9-e11 are register bits 3-5
#pragma unroll
    for (int h = 8; h < 64; h <<= 1)
#pragma unroll
      for (int r = 0; r < 64; ++r)
        if ((r & h) == 0) {
          const float a = v[r], b = v[r + h];
          v[r] = a + b;
          v[r + h] = a - b;
        }
    // exchange: element e lives in float4 slot x4096_slot(e / 4)
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 128 * t + 8 * n + 4 * h + g;
        slice[x4096_slot(c)] = make_float4(v[8 * t + 4 * h], v[8 * t + 4 * h + 1],
                                           v[8 * t + 4 * h + 2], v[8 * t + 4 * h + 3]);
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
    // phase 2 registers: r' = 8 k + i, k bits = (e5, e6, e7)
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = e2base + 32 * (k & 1) + 64 * ((k >> 1) & 1) + 128 * (k >> 2) + 4 * h;
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
#pragma unroll
    for (int r = 0; r < 64; ++r) v[r] = dpp_butterfly<kDppRowRor8>(v[r], s_r8);
    // scale: the transform is unnormalised; 1/sqrt(4096) = 1/64 is exact
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 64; ++r) amax = fmaxf(amax, fabsf(v[r]));
    amax = wave_max_dpp(amax) * (1.0f / 64.0f);
    const __half s16 = row_scale_fp16(amax, clip_ratio);
    const float kq = inv_scale(s16) * (1.0f / 64.0f);
    uint8_t* qrow = q_out + row * ld_q;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float t8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t8[i] = magic_code<CLAMP>(v[8 * k + i], kq);
      const int e0 = e2base + 32 * (k & 1) + 64 * ((k >> 1) & 1) + 128 * (k >> 2);
      *reinterpret_cast<uint32_t*>(qrow + (e0 >> 1)) = pack8_magic(t8);
    }
    if (lane == 0) scale_out[row] = s16;
    if (x_rot) {
      const float cn = 1.0f / 64.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e0 = e2base + 32 * (k & 1) + 64 * ((k >> 1) & 1) + 128 * (k >> 2);
        float4* dst = reinterpret_cast<float4*>(x_rot + row * 4096 + e0);
        dst[0] = make_float4(v[8 * k] * cn, v[8 * k + 1] * cn, v[8 * k + 2] * cn, v[8 * k + 3] * cn);
        dst[1] = make_float4(v[8 * k + 4] * cn, v[8 * k + 5] * cn, v[8 * k + 6] * cn,
                             v[8 * k + 7] * cn);
      }
    }
  }
}

}  // namespace quarot
