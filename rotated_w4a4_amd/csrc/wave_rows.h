// Wave-level helpers shared by the rotate+quant kernels: DPP moves, the
// wave-wide maximum and the MFMA operand vector types.
#pragma once

#include "quant_common.h"

namespace quarot {

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
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

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_mov<kDppQuadX1>(v);
  v += dpp_mov<kDppQuadX2>(v);
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

}  // namespace quarot
