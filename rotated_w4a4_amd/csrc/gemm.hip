// quarot_w4a4_gemm: INT4 x INT4 GEMM on CDNA4 int8 MFMA with INT32
// accumulation and the per-token x per-channel dequant epilogue.
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary), section 3.4 Stage 2b (Y_ij = acc_ij * scale_x[i] * scale_w[j])
// and "Kernel Implementation and Hardware Efficiency" (INT4 GEMM of packed
// activations against offline-packed weights, INT32 accumulator, dequant to
// FP16).  gfx950 has no INT4 matrix instruction, so each packed byte is
// widened to two int8 lanes.
//
// Widening.  A packed 32-bit word w holds 8 codes (code i in nibble i).
//   (w << 4) & 0xF0F0F0F0  -> bytes 16*q0, 16*q2, 16*q4, 16*q6
//    w       & 0xF0F0F0F0  -> bytes 16*q1, 16*q3, 16*q5, 16*q7
// (a nibble in the top half of a byte, low half zero, is 16x its two's
// complement value).  Both operands are widened with the same byte
// placement, so every MFMA pairs A and B values of the same K index; the
// accumulator holds 256 * acc exactly (256 * 64 * K <= 2^30 for K <= 65536)
// and the epilogue shifts it right by 8.
//
// Tiling.  Workgroup tile 128 (M) x 256 (N) x 128 (K), 4 waves of 64 x 128,
// each wave 2 x 4 blocks of v_mfma_i32_32x32x32_i8.  Packed tiles are staged
// in LDS (double buffered, rows padded to 80 bytes).  Each lane reads 16
// packed bytes per block and K-pair: the first 8 feed one MFMA, the last 8
// the next, so lane half h covers K offsets [32h, 32h + 32) of a 64-wide
// K-pair.  Tiles are assigned XCD-major: consecutive tile ids go to the same
// XCD so neighbouring tiles share its L2.
#include "common.h"

namespace quarot {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128;
constexpr int BN = 256;
constexpr int BK = 128;             // int4 elements per K tile
constexpr int BKB = BK / 2;         // bytes per row per K tile (64)
constexpr int LDS_STRIDE = 80;      // padded row stride in bytes
constexpr int kThreads = 256;
constexpr int A_CHUNKS = BM * BKB / 16 / kThreads;  // 16-byte loads per thread: 2
constexpr int B_CHUNKS = BN * BKB / 16 / kThreads;  // 4
constexpr int WM = 64, WN = 128;    // wave tile
constexpr int FM = WM / 32, FN = WN / 32;  // MFMA blocks per wave: 2 x 4
constexpr int GROUP_M = 4;

__device__ __forceinline__ void widen(const uint4& p, v4i& lo, v4i& hi) {
  lo[0] = int((p.x << 4) & 0xF0F0F0F0u);
  lo[1] = int(p.x & 0xF0F0F0F0u);
  lo[2] = int((p.y << 4) & 0xF0F0F0F0u);
  lo[3] = int(p.y & 0xF0F0F0F0u);
  hi[0] = int((p.z << 4) & 0xF0F0F0F0u);
  hi[1] = int(p.z & 0xF0F0F0F0u);
  hi[2] = int((p.w << 4) & 0xF0F0F0F0u);
  hi[3] = int(p.w & 0xF0F0F0F0u);
}

__global__ __launch_bounds__(kThreads) void w4a4_gemm_kernel(
    const uint8_t* __restrict__ a_q, int64_t lda, const __half* __restrict__ a_scale,
    const uint8_t* __restrict__ b_q, int64_t ldb, const __half* __restrict__ b_scale,
    int M, int N, int K, __half* __restrict__ c, int64_t ldc, int32_t* __restrict__ acc_out,
    int64_t ld_acc, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][(BM + BN) * LDS_STRIDE];

  // --- tile assignment: XCD-major, then grouped along M -------------------
  const int total = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
  const int group = pid / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (pid % (GROUP_M * tiles_n)) % gsz;
  const int tn = (pid % (GROUP_M * tiles_n)) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = (wave >> 1) * WM;  // wave row offset inside the tile
  const int wn = (wave & 1) * WN;   // wave col offset inside the tile
  const int kbytes = K >> 1;

  // global -> register staging of one K tile
  uint4 ra[A_CHUNKS], rb[B_CHUNKS];
  auto load_tile = [&](int kt) {
    const int kb0 = kt * BKB;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int cidx = tid + i * kThreads;
      const int row = cidx >> 2, col = (cidx & 3) * 16;
      const int gr = min(m0 + row, M - 1);
      if (kb0 + col < kbytes)
        ra[i] = *reinterpret_cast<const uint4*>(a_q + int64_t(gr) * lda + kb0 + col);
      else
        ra[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      const int cidx = tid + i * kThreads;
      const int row = cidx >> 2, col = (cidx & 3) * 16;
      const int gr = min(n0 + row, N - 1);
      if (kb0 + col < kbytes)
        rb[i] = *reinterpret_cast<const uint4*>(b_q + int64_t(gr) * ldb + kb0 + col);
      else
        rb[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int cidx = tid + i * kThreads;
      const int row = cidx >> 2, col = (cidx & 3) * 16;
      *reinterpret_cast<uint4*>(&smem[buf][row * LDS_STRIDE + col]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      const int cidx = tid + i * kThreads;
      const int row = cidx >> 2, col = (cidx & 3) * 16;
      *reinterpret_cast<uint4*>(&smem[buf][(BM + row) * LDS_STRIDE + col]) = rb[i];
    }
  };

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16i{};

  const int ktiles = (K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int frow = lane & 31;       // row (A) / column (B) of the fragment
  const int fcol = (lane >> 5) * 16;  // byte offset of this lane half in a K-pair

  for (int kt = 0; kt < ktiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ktiles) load_tile(kt + 1);
    const uint8_t* sa = &smem[buf][0];
    const uint8_t* sb = &smem[buf][BM * LDS_STRIDE];
#pragma unroll
    for (int kp = 0; kp < BKB / 32; ++kp) {  // two 64-wide K-pairs per tile
      v4i alo[FM], ahi[FM], blo[FN], bhi[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint4 p = *reinterpret_cast<const uint4*>(
            sa + (wm + i * 32 + frow) * LDS_STRIDE + kp * 32 + fcol);
        widen(p, alo[i], ahi[i]);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint4 p = *reinterpret_cast<const uint4*>(
            sb + (wn + j * 32 + frow) * LDS_STRIDE + kp * 32 + fcol);
        widen(p, blo[j], bhi[j]);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo[i], blo[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi[i], bhi[j], acc[i][j], 0, 0, 0);
        }
    }
    if (kt + 1 < ktiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // --- epilogue: acc / 256 -> fp32 * scale_x * scale_w -> fp16 -----------
  // 32x32 block layout: lane holds column (lane & 31); register r holds row
  // 8 * (r / 4) + 4 * (lane / 32) + (r % 4).
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = n0 + wn + j * 32 + (lane & 31);
    const bool col_ok = col < N;
    const float sw = col_ok ? __half2float(b_scale[col]) : 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (!col_ok || row >= M) continue;
        const int32_t v = acc[i][j][r] >> 8;
        const float sx = __half2float(a_scale[row]);
        c[int64_t(row) * ldc + col] = __float2half_rn((float(v) * sx) * sw);
        if (acc_out) acc_out[int64_t(row) * ld_acc + col] = v;
      }
    }
  }
}

}  // namespace

int launch_w4a4_gemm(const uint8_t* a_q, int64_t lda, const __half* a_scale,
                     const uint8_t* b_q, int64_t ldb, const __half* b_scale,
                     int64_t M, int64_t N, int64_t K, __half* c, int64_t ldc,
                     int32_t* acc_out, int64_t ld_acc, hipStream_t stream) {
  const int tiles_m = int((M + BM - 1) / BM);
  const int tiles_n = int((N + BN - 1) / BN);
  const int64_t total = int64_t(tiles_m) * tiles_n;
  if (total > 0x7fffffff) {
    set_error("too many tiles");
    return QUAROT_ERR_UNSUPPORTED;
  }
  hipLaunchKernelGGL(w4a4_gemm_kernel, dim3(unsigned(total)), dim3(kThreads), 0, stream, a_q,
                     lda, a_scale, b_q, ldb, b_scale, int(M), int(N), int(K), c, ldc, acc_out,
                     ld_acc, tiles_m, tiles_n);
  return check_launch("w4a4_gemm");
}

}  // namespace quarot
