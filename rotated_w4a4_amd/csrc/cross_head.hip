// Cross-head transform + per-token INT4 quantisation of the attention output
// (the input of the out-projection).
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary), section 3.4 Stage 1c: the head-wise factor I_{n_h} (x) H_{d_h} of
// the full Hadamard is folded into W_v and W_out offline, and the remaining
// factor is applied online to the concatenated attention output,
// Z <- Z (H_{n_h} (x) I_{d_h}): a length-n_h Walsh-Hadamard transform over the
// head index for each head-dim lane.  Stage 2b then quantises each token
// symmetrically (S = clip * max|z~| / 7) for the INT4 out-projection.
//
// Layout.  One wave owns one row of n_h * 128 fp16 values.  Lane l holds
// lanes 2l and 2l + 1 of every head (one 4-byte load per head; the 64 lanes
// of a load instruction read one head's 256 contiguous bytes), so the whole
// transform runs on registers: log2(n_h) butterfly stages over the head
// index, no LDS and no cross-lane exchange except the row maximum.  Each
// lane's two codes of a head form one byte (even lane in the low nibble):
// 64 contiguous bytes per store instruction.
#include "cross_head.h"
#include "wave_rows.h"

namespace quarot {
namespace {

constexpr int kHeadDim = 128;
constexpr int kRowsPerBlock = 4;  // one wave per row
constexpr int64_t kMaxBlocks = int64_t(1) << 16;

template <int NH>
__device__ __forceinline__ constexpr float head_norm() {
  // 1 / sqrt(NH) for NH = 2^k
  return NH == 1 ? 1.0f
         : NH == 2 ? 0.70710678118654752f
         : NH == 4 ? 0.5f
         : NH == 8 ? 0.35355339059327376f
         : NH == 16 ? 0.25f
         : NH == 32 ? 0.17677669529663688f
                    : 0.125f;
}

// One row on one wave.
template <int NH, bool CLAMP>
__device__ __forceinline__ void cross_head_row(const __half* __restrict__ z, int64_t row,
                                               int64_t ld_z, float clip_ratio,
                                               uint8_t* __restrict__ q_out, int64_t ld_q,
                                               __half* __restrict__ scale_out,
                                               float* __restrict__ z_rot, int lane) {
  const __half* src = z + row * ld_z + 2 * lane;

  uint32_t raw[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) raw[h] = *reinterpret_cast<const uint32_t*>(src + h * kHeadDim);

  float v0[NH], v1[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const float2 f = __half22float2(__builtin_bit_cast(__half2, raw[h]));
    v0[h] = f.x;
    v1[h] = f.y;
  }
  // unnormalised Sylvester transform over the head index
#pragma unroll
  for (int s = 1; s < NH; s <<= 1) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      if ((h & s) == 0) {
        const float a0 = v0[h], b0 = v0[h + s];
        const float a1 = v1[h], b1 = v1[h + s];
        v0[h] = a0 + b0;
        v0[h + s] = a0 - b0;
        v1[h] = a1 + b1;
        v1[h + s] = a1 - b1;
      }
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int h = 0; h < NH; ++h) amax = fmaxf(amax, fmaxf(fabsf(v0[h]), fabsf(v1[h])));
  amax = wave_max_dpp(amax);

  constexpr float kNorm = head_norm<NH>();
  const __half s16 = row_scale_fp16(amax * kNorm, clip_ratio);
  const float kq = inv_scale(s16) * kNorm;
  uint8_t* qrow = q_out + row * ld_q + lane;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const uint32_t c0 = __builtin_bit_cast(uint32_t, magic_code<CLAMP>(v0[h], kq));
    const uint32_t c1 = __builtin_bit_cast(uint32_t, magic_code<CLAMP>(v1[h], kq));
    // byte 0 of each is q + 8; xor 8 gives the 4-bit two's complement
    qrow[h * (kHeadDim / 2)] = static_cast<uint8_t>((((c1 << 4) | (c0 & 0xFu)) ^ 0x88u) & 0xFFu);
  }
  if (lane == 0) scale_out[row] = s16;
  if (z_rot) {
    float2* dst = reinterpret_cast<float2*>(z_rot + row * (NH * kHeadDim) + 2 * lane);
#pragma unroll
    for (int h = 0; h < NH; ++h) dst[h * (kHeadDim / 2)] = make_float2(v0[h] * kNorm, v1[h] * kNorm);
  }
}

// One wave per row.  With LOOP (launches of more rows than four times the
// capped grid) the waves stride over further rows; rows are uniform per wave
// and no barrier follows, so each wave loops on its own.  The single-row
// form is kept for every other launch: the loop measured about 5% slower at
// 64 heads.
template <int NH, bool CLAMP, bool LOOP>
__global__ __launch_bounds__(64 * kRowsPerBlock) void cross_head_quant_kernel(
    const __half* __restrict__ z, int64_t rows, int64_t ld_z, float clip_ratio,
    uint8_t* __restrict__ q_out, int64_t ld_q, __half* __restrict__ scale_out,
    float* __restrict__ z_rot) {
  const int lane = threadIdx.x & 63;
  int64_t row = int64_t(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (LOOP) {
    const int64_t stride = int64_t(gridDim.x) * kRowsPerBlock;
    for (; row < rows; row += stride)
      cross_head_row<NH, CLAMP>(z, row, ld_z, clip_ratio, q_out, ld_q, scale_out, z_rot, lane);
  } else if (row < rows) {
    cross_head_row<NH, CLAMP>(z, row, ld_z, clip_ratio, q_out, ld_q, scale_out, z_rot, lane);
  }
}

template <int NH>
int launch_nh(const __half* z, int64_t rows, int64_t ld_z, float clip_ratio, uint8_t* q_out,
              int64_t ld_q, __half* scale_out, float* z_rot, hipStream_t stream) {
  // at most 2^16 blocks (the waves loop over further rows), so the grid's
  // work-item count stays far below 2^32
  const int64_t blocks = std::min<int64_t>((rows + kRowsPerBlock - 1) / kRowsPerBlock, kMaxBlocks);
  const dim3 grid(static_cast<unsigned>(blocks));
  const dim3 block(64 * kRowsPerBlock);
  const bool loop = blocks * kRowsPerBlock < rows;
#define QR_CH(CL, LP)                                                                            \
  hipLaunchKernelGGL((cross_head_quant_kernel<NH, CL, LP>), grid, block, 0, stream, z, rows, ld_z, \
                     clip_ratio, q_out, ld_q, scale_out, z_rot)
  if (clip_ratio < 1.0f) {
    if (loop) QR_CH(true, true); else QR_CH(true, false);
  } else {
    if (loop) QR_CH(false, true); else QR_CH(false, false);
  }
#undef QR_CH
  return check_launch("cross_head_quant_kernel");
}

}  // namespace

int launch_cross_head_quant(const __half* z, int64_t rows, int n_heads, int64_t ld_z,
                            float clip_ratio, uint8_t* q_out, int64_t ld_q, __half* scale_out,
                            float* z_rot, hipStream_t stream) {
  switch (n_heads) {
    case 1: return launch_nh<1>(z, rows, ld_z, clip_ratio, q_out, ld_q, scale_out, z_rot, stream);
    case 2: return launch_nh<2>(z, rows, ld_z, clip_ratio, q_out, ld_q, scale_out, z_rot, stream);
    case 4: return launch_nh<4>(z, rows, ld_z, clip_ratio, q_out, ld_q, scale_out, z_rot, stream);
    case 8: return launch_nh<8>(z, rows, ld_z, clip_ratio, q_out, ld_q, scale_out, z_rot, stream);
    case 16: return launch_nh<16>(z, rows, ld_z, clip_ratio, q_out, ld_q, scale_out, z_rot, stream);
    case 32: return launch_nh<32>(z, rows, ld_z, clip_ratio, q_out, ld_q, scale_out, z_rot, stream);
    case 64: return launch_nh<64>(z, rows, ld_z, clip_ratio, q_out, ld_q, scale_out, z_rot, stream);
    default:
      set_error("n_heads = %d: supported counts are 1, 2, 4, ..., 64", n_heads);
      return QUAROT_ERR_UNSUPPORTED;
  }
}

}  // namespace quarot
