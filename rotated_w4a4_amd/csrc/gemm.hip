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
// Tiling.  Workgroup tile BM x BN x 128 (K), waves of WM x WN, each wave
// (WM/32) x (WN/32) blocks of v_mfma_i32_32x32x32_i8.  Packed tiles are
// staged in LDS (two buffers, 16-byte chunks XOR-swizzled per row); two more
// tiles are in flight into registers, so global loads are issued two tiles
// ahead of use and each K step has a single barrier.  Each lane reads 16
// packed bytes per block and K-pair: the first 8 feed one MFMA, the last 8
// the next, so lane half h covers K offsets [32h, 32h + 32) of a 64-wide
// K-pair.  Tiles are assigned XCD-major:
// consecutive tile ids go to the same XCD so neighbouring tiles share its L2.
#include "common.h"

namespace quarot {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int GROUP_M = 4;

// LDS holds one K tile per buffer, row-major with BKB-byte rows (no
// padding).  The LDS has 64 four-byte banks and serves a 128-bit read for 16
// lanes per cycle, so the 16 rows a fragment read touches (same logical
// 16-byte chunk) must land in 16 different 16-byte slots of a 256-byte bank
// period.  Chunk c of row r is stored at chunk slot c ^ swz(r); with 64-byte
// rows (4 chunks) swz(r) = ((r >> 1) ^ (r >> 3)) & 3, with 128-byte rows
// (8 chunks) swz(r) = (r >> 1) & 7.  The cooperative stores write whole rows
// and stay conflict-free.
template <int BKB>
__device__ __forceinline__ int lds_off(int r, int c) {
  constexpr int CPR = BKB / 16;
  const int sw = (CPR == 4) ? (((r >> 1) ^ (r >> 3)) & 3) : ((r >> 1) & (CPR - 1));
  return r * BKB + ((c ^ sw) << 4);
}

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

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <int WAVES_M_, int WAVES_N_, int WM_, int WN_, int BK_>
struct GemmCfg {
  static constexpr int BK = BK_;                  // int4 elements per K tile
  static constexpr int BKB = BK / 2;              // bytes per row per K tile
  static constexpr int CPR = BKB / 16;            // 16-byte chunks per row
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int BM = WAVES_M * WM, BN = WAVES_N * WN;
  static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int ROWS = BM + BN;            // A rows then B rows of a tile
  static constexpr int CH = ROWS * CPR / THREADS;  // 16-byte chunks per thread per tile
  static constexpr int ROWS_PER_PASS = THREADS / CPR;
  static constexpr int STAGE = ROWS * BKB;
  static_assert(ROWS * CPR % THREADS == 0, "tile rows must split evenly over threads");
  static_assert(BM % ROWS_PER_PASS == 0, "a load pass must not straddle A and B");
};

// 8 waves of 64 x 64: BM = 128, BN = 256, two waves per SIMD; K tile 256.
using Cfg8 = GemmCfg<2, 4, 64, 64, 256>;

template <class C>
__global__ __launch_bounds__(C::THREADS) void w4a4_gemm_kernel(
    const uint8_t* __restrict__ a_q, int64_t lda, const __half* __restrict__ a_scale,
    const uint8_t* __restrict__ b_q, int64_t ldb, const __half* __restrict__ b_scale,
    int M, int N, int K, __half* __restrict__ c, int64_t ldc, int32_t* __restrict__ acc_out,
    int64_t ld_acc, int tiles_m, int tiles_n) {
  constexpr int FM = C::FM, FN = C::FN, CH = C::CH, BM = C::BM, BN = C::BN;
  constexpr int BKB = C::BKB, CPR = C::CPR;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][C::STAGE];

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
  const int wm = (wave / C::WAVES_N) * C::WM;  // wave row offset inside the tile
  const int wn = (wave % C::WAVES_N) * C::WN;  // wave col offset inside the tile
  const int kbytes = K >> 1;

  // Thread tid moves chunk (tid % CPR) of tile rows tid / CPR +
  // ROWS_PER_PASS * i (A rows first, then B rows); rows past the matrix edge
  // re-read the last row (their results are never stored).
  const int lrow = tid / CPR, lchunk = tid % CPR;
  const uint8_t* src[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int r = lrow + C::ROWS_PER_PASS * i;
    src[i] = (r < BM) ? a_q + int64_t(min(m0 + r, M - 1)) * lda + 16 * lchunk
                      : b_q + int64_t(min(n0 + r - BM, N - 1)) * ldb + 16 * lchunk;
  }
  const int kfull = kbytes / BKB;  // tiles entirely inside K
  const bool has_tail = (kbytes % BKB) != 0;

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16i{};

  const int frow = lane & 31;   // row (A) / column (B) of the fragment
  const int fhalf = lane >> 5;  // which 16-byte chunk of a 32-byte K-pair
  // All fragment reads of a tile are issued before its MFMAs so the LDS
  // latency overlaps the first MFMAs instead of stalling each K-pair.
  constexpr int KP = BKB / 32;  // 64-wide K-pairs per tile
  auto compute_tile = [&](int buf) {
    const uint8_t* sa = smem[buf];
    const uint8_t* sb = smem[buf] + BM * BKB;
    uint4 fa[KP][FM], fb[KP][FN];
#pragma unroll
    for (int kp = 0; kp < KP; ++kp) {
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[kp][i] = ld16(sa + lds_off<BKB>(wm + i * 32 + frow, 2 * kp + fhalf));
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[kp][j] = ld16(sb + lds_off<BKB>(wn + j * 32 + frow, 2 * kp + fhalf));
    }
#pragma unroll
    for (int kp = 0; kp < KP; ++kp) {
      v4i alo[FM], ahi[FM], blo[FN], bhi[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) widen(fa[kp][i], alo[i], ahi[i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) widen(fb[kp][j], blo[j], bhi[j]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo[i], blo[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi[i], bhi[j], acc[i][j], 0, 0, 0);
        }
    }
  };

  // Pipeline over the full tiles: tile kt is computed from one LDS buffer,
  // then tile kt+1 goes from registers into the other buffer while tiles
  // kt+2 and kt+3 are in flight from memory.  The loop is unrolled by two
  // so each register set keeps a fixed role, and loads are issued every step
  // (past the end they re-read the last full tile) so every path through the
  // loop has the same wait counts.
  uint4 r0[CH], r1[CH];
#define QR_LOAD(r, kb0)                                          \
  _Pragma("unroll") for (int i = 0; i < CH; ++i) r[i] = ld16(src[i] + (kb0))
#define QR_STORE(buf, r)                                                                  \
  _Pragma("unroll") for (int i = 0; i < CH; ++i) *reinterpret_cast<uint4*>(               \
      smem[buf] + lds_off<BKB>(lrow + C::ROWS_PER_PASS * i, lchunk)) = r[i]
  if (kfull > 0) {
    // Step i: compute tile i from buffer i % 2, store tile i+1 (in registers
    // since step i-2) into the other buffer, issue the loads of tile i+3 into
    // the registers just freed, one barrier.  sched_barrier keeps that order.
    QR_LOAD(r0, 0);
    QR_LOAD(r1, min(1, kfull - 1) * BKB);
    QR_STORE(0, r0);
    QR_LOAD(r0, min(2, kfull - 1) * BKB);
    __syncthreads();
    int kt = 0;
    for (; kt + 2 <= kfull; kt += 2) {
      compute_tile(0);  // tile kt
      __builtin_amdgcn_sched_barrier(0);
      QR_STORE(1, r1);  // tile kt+1
      QR_LOAD(r1, min(kt + 3, kfull - 1) * BKB);
      __syncthreads();
      compute_tile(1);  // tile kt+1
      __builtin_amdgcn_sched_barrier(0);
      QR_STORE(0, r0);  // tile kt+2 (a harmless repeat past the end)
      QR_LOAD(r0, min(kt + 4, kfull - 1) * BKB);
      __syncthreads();
    }
    if (kt < kfull) compute_tile(0);  // odd count: the last full tile is in buffer 0
  }
  if (has_tail) {  // the partial tile at the end of K: chunks past K read as zero
    __syncthreads();
    const int kb0 = kfull * BKB;
    const bool ok = kb0 + 16 * lchunk < kbytes;
    QR_LOAD(r0, ok ? kb0 : 0);
#pragma unroll
    for (int i = 0; i < CH; ++i) r0[i] = ok ? r0[i] : make_uint4(0, 0, 0, 0);
    QR_STORE(1, r0);
    __syncthreads();
    compute_tile(1);
  }
#undef QR_LOAD
#undef QR_STORE

  // --- epilogue: acc / 256 -> fp32 * scale_x * scale_w -> fp16 -----------
  // 32x32 block layout: lane holds column (lane & 31); register r holds row
  // 8 * (r / 4) + 4 * (lane / 32) + (r % 4).
  float sx[FM][16];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      sx[i][r] = __half2float(a_scale[min(row, M - 1)]);
    }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = n0 + wn + j * 32 + (lane & 31);
    const bool col_ok = col < N;
    const float sw = __half2float(b_scale[min(col, N - 1)]);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (!col_ok || row >= M) continue;
        const int32_t v = acc[i][j][r] >> 8;
        c[int64_t(row) * ldc + col] = __float2half_rn((float(v) * sx[i][r]) * sw);
        if (acc_out) acc_out[int64_t(row) * ld_acc + col] = v;
      }
    }
  }
}

template <class C>
int launch_cfg(const uint8_t* a_q, int64_t lda, const __half* a_scale, const uint8_t* b_q,
               int64_t ldb, const __half* b_scale, int64_t M, int64_t N, int64_t K, __half* c,
               int64_t ldc, int32_t* acc_out, int64_t ld_acc, hipStream_t stream) {
  const int tiles_m = int((M + C::BM - 1) / C::BM);
  const int tiles_n = int((N + C::BN - 1) / C::BN);
  const int64_t total = int64_t(tiles_m) * tiles_n;
  if (total > 0x7fffffff) {
    set_error("too many tiles");
    return QUAROT_ERR_UNSUPPORTED;
  }
  hipLaunchKernelGGL(w4a4_gemm_kernel<C>, dim3(unsigned(total)), dim3(C::THREADS), 0, stream,
                     a_q, lda, a_scale, b_q, ldb, b_scale, int(M), int(N), int(K), c, ldc,
                     acc_out, ld_acc, tiles_m, tiles_n);
  return check_launch("w4a4_gemm");
}

}  // namespace

int launch_w4a4_gemm(const uint8_t* a_q, int64_t lda, const __half* a_scale,
                     const uint8_t* b_q, int64_t ldb, const __half* b_scale,
                     int64_t M, int64_t N, int64_t K, __half* c, int64_t ldc,
                     int32_t* acc_out, int64_t ld_acc, hipStream_t stream) {
  return launch_cfg<Cfg8>(a_q, lda, a_scale, b_q, ldb, b_scale, M, N, K, c, ldc, acc_out,
                          ld_acc, stream);
}

}  // namespace quarot
