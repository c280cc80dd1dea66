// Rotate+quant of rows of d = 4096: two waves share one row.
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary), section 3.4 Stage 1a (R = H diag(s)), Stage 1b (online Hadamard
// in FP32) and Stage 2b (per-token symmetric INT4); "QuaRot Guide",
// section 3 of "The Architecture" (the fast transform).
//
// A row is 4096 fp16 values (8 KiB).  With one wave per row the compute of
// the rows whose data arrives last is a long serial tail, so the row is
// split over the two waves of a 128-thread workgroup (all 2048 rows of a
// prefill batch are resident at once, four waves per SIMD).  Element bits
// e0 .. e11 are handed out as follows:
//   phase 1  wave w, lane n + 16 g, tile t (0..3): elements
//            512 (4 w + t) + 32 n + 8 g + (0..7) are the B operand of
//            v_mfma_f32_16x16x32_f16; two MFMAs with rows 0-15 and 16-31 of
//            the Sylvester H_32 as A transform e0-e4 exactly (products with
//            +-1, fp32 sums).  The output element 512 (4 w + t) + 32 n +
//            16 h + 4 g + i sits in register 8 t + 4 h + i.  Butterflies:
//            e9, e10 (tile bits) in registers; e5, e6, e8 (lane bits 0, 1,
//            3) by DPP.  The row goes to LDS as fp32.
//   phase 2  wave w' = e10, lane = (e3, e4, e5, e6, e8, e9), register
//            bits = (e0, e1, e2, e7, e11): a lane holds runs of eight
//            consecutive elements (two float4 reads each).  Butterflies over
//            e7 and e11 in registers, the row max over the workgroup, then
//            each lane packs a run's eight codes into one 32-bit word: four
//            stores of 256 consecutive bytes per wave.
#pragma once

#include "wave_rows.h"

namespace quarot {

constexpr int kSplitBlock = 128;  // two waves, one row

// Float4 slot of chunk c (= element / 4) in the row's LDS copy: c with bits
// 0-2 XORed with parities of higher bits (bit 0 with c5 ^ c6, bit 1 with
// c3 ^ c4 ^ c7, bit 2 with c3 ^ c6 ^ c8), a bijection since the higher bits
// stay.  Neither the phase-1 writes (chunks 128 (4 w + t) + 8 n + 4 h + g)
// nor the phase-2 reads (chunks 2 (lane & 15) + 64 (lane >> 4) + const)
// count bank-conflict cycles with it: a read/write probe of both patterns
// (SQ_LDS_BANK_CONFLICT) found it among random swizzles of this form.  The
// earlier c ^ ((c >> 4) & 7), chosen on a model of 16 lanes per 128-bit LDS
// cycle, left the writes heavily conflicted.
__device__ __forceinline__ constexpr int split_slot(int c) {
  return c ^ ((((c >> 5) ^ (c >> 6)) & 1) | ((((c >> 3) ^ (c >> 4) ^ (c >> 7)) & 1) << 1) |
              ((((c >> 3) ^ (c >> 6) ^ (c >> 8)) & 1) << 2));
}
// An access's chunk is c = a + b with a lane part a (computed once) and a
// part b fixed at compile time (the unrolled register index), their bits
// disjoint.  The XOR term is linear over GF(2) in bits 3-8 and lands in bits
// 0-2, so split_slot(a + b) = (split_slot(a) ^ (split_slot(b) & 7)) +
// (b & ~7): one XOR with a constant per access, and the add folds into the
// LDS instruction's offset.
__device__ __forceinline__ int split_slot_at(int slot_a, int b) {
  return (slot_a ^ (split_slot(b) & 7)) + (b & ~7);
}

// One DPP butterfly stage over lane bit 0, 1 or 3 (STAGE 0, 1, 2) on 32
// registers, as v + partner * c in one v_fmac_f32 with DPP (c = +1 on the
// low lane, -1 on the high lane: a high lane ends with b - a, a sign the
// caller tracks).  Every block opens with s_nop 1 (two wait states between
// a VALU write of a source and its DPP read) and the last stage closes with
// one.
template <int STAGE>
__device__ __forceinline__ void split_dpp_stage(float (&v)[32], float c) {
#define QR_FMAC_DPP4(CTRL, TRAIL)                                                           \
  asm volatile("s_nop 1\n"                                                                  \
               "v_fmac_f32_dpp %0, %0, %4 " CTRL " row_mask:0xf bank_mask:0xf\n"          \
               "v_fmac_f32_dpp %1, %1, %4 " CTRL " row_mask:0xf bank_mask:0xf\n"          \
               "v_fmac_f32_dpp %2, %2, %4 " CTRL " row_mask:0xf bank_mask:0xf\n"          \
               "v_fmac_f32_dpp %3, %3, %4 " CTRL " row_mask:0xf bank_mask:0xf" TRAIL      \
               : "+v"(v[r]), "+v"(v[r + 1]), "+v"(v[r + 2]), "+v"(v[r + 3])               \
               : "v"(c))
#pragma unroll
  for (int r = 0; r < 32; r += 4) {
    if (STAGE == 0) QR_FMAC_DPP4("quad_perm:[1,0,3,2]", "");
    else if (STAGE == 1) QR_FMAC_DPP4("quad_perm:[2,3,0,1]", "");
    else if (r != 28) QR_FMAC_DPP4("row_ror:8", "");
    else QR_FMAC_DPP4("row_ror:8", "\ns_nop 1");
  }
#undef QR_FMAC_DPP4
}

template <bool CLAMP>
__global__ __launch_bounds__(kSplitBlock, 4) void had_quant_4096_split(
    const __half* __restrict__ x, int64_t rows, int64_t ld_x, const int8_t* __restrict__ signs,
    float clip_ratio, uint8_t* __restrict__ q_out, int64_t ld_q, __half* __restrict__ scale_out,
    float* __restrict__ x_rot) {
  __shared__ float4 lds[1024];
  __shared__ float red[kSplitBlock / 64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int e_in = 2048 * wave + 32 * n + 8 * g;  // tile t adds 512 t
  const float c0 = (lane & 1) ? -1.0f : 1.0f;
  const float c1 = (lane & 2) ? -1.0f : 1.0f;
  const float c3 = (lane & 8) ? -1.0f : 1.0f;
  // phase 2: e3-e6 = lane bits 0-3, e8, e9 = lane bits 4, 5, e10 = the wave;
  // the DPP stages left the sign (-1)^(e5 + e6 + e8) on every value of the lane
  const int e2 = 8 * (lane & 15) + 256 * (lane >> 4) + 1024 * wave;
  const float sigma = ((((lane >> 2) ^ (lane >> 3) ^ (lane >> 4)) & 1) != 0) ? -1.0f : 1.0f;
  // LDS slots of the lane parts of the phase-1 chunks (512 w + 8 n + g) and
  // of the phase-2 chunks (e2 / 4); the register index adds the fixed part
  const int slot_w = split_slot(512 * wave + 8 * n + g);
  const int slot_r = split_slot(e2 >> 2);

  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const __half* src = x + row * ld_x + e_in;
    uint4 raw[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) raw[t] = *reinterpret_cast<const uint4*>(src + 512 * t);
    // sign masks and H_32 rows n, n + 16 (columns 8 g + j), rebuilt per row
    // (a block normally does one row; keeping them would cost registers)
    uint4 mask[4];
    if (signs) {
      uint2 w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = *reinterpret_cast<const uint2*>(signs + e_in + 512 * t);
#pragma unroll
      for (int t = 0; t < 4; ++t) mask[t] = sign_masks8(w[t].x, w[t].y);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) mask[t] = make_uint4(0, 0, 0, 0);
    }
    half8_t h_lo, h_hi;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = 8 * g + j;
      h_lo[j] = (__builtin_popcount(n & k) & 1) ? _Float16(-1.0f) : _Float16(1.0f);
      h_hi[j] = (__builtin_popcount((n + 16) & k) & 1) ? _Float16(-1.0f) : _Float16(1.0f);
    }
    // ---- phase 1 -------------------------------------------------------
    float v[32];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
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
#pragma unroll
    for (int h = 8; h < 32; h <<= 1)  // e9, e10
#pragma unroll
      for (int r = 0; r < 32; ++r)
        if ((r & h) == 0) {
          const float a = v[r], b = v[r + h];
          v[r] = a + b;
          v[r + h] = a - b;
        }
    split_dpp_stage<0>(v, c0);  // e5
    split_dpp_stage<1>(v, c1);  // e6
    split_dpp_stage<2>(v, c3);  // e8
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // chunk 128 (4 w + t) + 8 n + 4 h + g
        lds[split_slot_at(slot_w, 128 * t + 4 * h)] = make_float4(v[8 * t + 4 * h], v[8 * t + 4 * h + 1],
                                         v[8 * t + 4 * h + 2], v[8 * t + 4 * h + 3]);
      }
    __syncthreads();
    // ---- phase 2: register r = e0 + 2 e1 + 4 e2 + 8 e7 + 16 e11 ----------
    // run u = e7 + 2 e11 starts at element e2 + 128 e7 + 2048 e11
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int u = k >> 1;
      // element e2 + 128 (u & 1) + 2048 (u >> 1) + 4 (k & 1)
      const float4 f = lds[split_slot_at(slot_r, 32 * (u & 1) + 512 * (u >> 1) + (k & 1))];
      v[4 * k] = f.x;
      v[4 * k + 1] = f.y;
      v[4 * k + 2] = f.z;
      v[4 * k + 3] = f.w;
    }
#pragma unroll
    for (int h = 8; h < 32; h <<= 1)  // e7 (h = 8), e11 (h = 16)
#pragma unroll
      for (int r = 0; r < 32; ++r)
        if ((r & h) == 0) {
          const float a = v[r], b = v[r + h];
          v[r] = a + b;
          v[r + h] = a - b;
        }
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 32; ++r) amax = fmaxf(amax, fabsf(v[r]));
    amax = wave_max_dpp(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();  // phase-2 reads done, red complete
    // the transform is unnormalised: 1/sqrt(4096) = 1/64 is exact
    amax = fmaxf(red[0], red[1]) * (1.0f / 64.0f);
    const __half s16 = row_scale_fp16(amax, clip_ratio);
    const float kq = inv_scale(s16) * (1.0f / 64.0f) * sigma;
    uint8_t* qrow = q_out + row * ld_q;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = magic_code<CLAMP>(v[8 * u + i], kq);
      const int e = e2 + 128 * (u & 1) + 2048 * (u >> 1);
      *reinterpret_cast<uint32_t*>(qrow + (e >> 1)) = pack8_magic(t);
    }
    if (threadIdx.x == 0) scale_out[row] = s16;
    if (x_rot) {
      const float cn = (1.0f / 64.0f) * sigma;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int u = k >> 1;
        const int e = e2 + 128 * (u & 1) + 2048 * (u >> 1) + 4 * (k & 1);
        *reinterpret_cast<float4*>(x_rot + row * 4096 + e) =
            make_float4(v[4 * k] * cn, v[4 * k + 1] * cn, v[4 * k + 2] * cn, v[4 * k + 3] * cn);
      }
    }
    __syncthreads();  // lds and red are reused by the next row
  }
}

}  // namespace quarot
