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
// Tiling.  Workgroup tile BM x BN x 256 (K), waves of WM x WN, each wave
// (WM/32) x (WN/32) blocks of v_mfma_i32_32x32x32_i8.  Packed tiles go from
// global memory straight into LDS (three stages, 16-byte chunks
// XOR-swizzled per row), two tiles ahead of use, with a single barrier per K
// tile.  The epilogue stages the accumulators through LDS so the fp16
// output leaves in 16-byte row segments.  Each lane reads 16
// packed bytes per block and K-pair: the first 8 feed one MFMA, the last 8
// the next, so lane half h covers K offsets [32h, 32h + 32) of a 64-wide
// K-pair.  Tiles are assigned XCD-major:
// consecutive tile ids go to the same XCD so neighbouring tiles share its L2.
#include "common.h"

namespace quarot {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Tiles are taken in groups of GROUP_M along M. With the XCD-major order an
// XCD's share of a 2048 x 4096 launch is then 8 x 4 tiles of 128 x 256
// (1024 A rows and 1024 B rows through its L2), not 4 x 8 (512 and 2048).
constexpr int GROUP_M = 8;

// LDS holds one K tile per buffer, row-major with BKB-byte rows (no
// padding).  The LDS has 64 four-byte banks, a 256-byte period.  Chunk c of
// row r is stored at chunk slot c ^ swz(r), where swz(r) is the index of the
// row's 256-byte period, taken modulo the chunks per row: (r >> 2) & 3 for
// 64-byte rows (4 chunks), (r >> 1) & 7 for 128-byte rows (8 chunks).  A
// fragment read (32 consecutive rows, one logical chunk per 32 lanes) then
// counts no bank-conflict cycles with either row length (SQ_LDS_BANK_CONFLICT
// on a read-only probe of each pattern; the 64-byte swizzle
// ((r >> 1) ^ (r >> 3)) & 3 counted 1.33 cycles per read).  The cooperative
// stores write whole rows and stay conflict-free.
template <int CPR>
__device__ __forceinline__ int lds_swz(int r) {
  static_assert(CPR == 4 || CPR == 8, "64- or 128-byte rows");
  return CPR == 4 ? ((r >> 2) & 3) : ((r >> 1) & 7);
}

template <int BKB>
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * BKB + ((c ^ lds_swz<BKB / 16>(r)) << 4);
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

// Byte address of a __shared__ object inside the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  typedef __attribute__((address_space(3))) const uint8_t lds_byte;
  return uint32_t(reinterpret_cast<uintptr_t>((lds_byte*)(p)));
}

// 16 bytes per lane from global memory straight into LDS at
// lds + 16 * lane (global_load_lds_dwordx4; the LDS base goes through M0,
// which needs one wait state before the load).  Completion is counted by
// vmcnt; the kernel below uses no other vector-memory loads while copies
// are in flight.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const uint8_t* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

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
  __shared__ __attribute__((aligned(16))) uint8_t smem[3][C::STAGE];

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int wm = (wave / C::WAVES_N) * C::WM;  // wave row offset inside the tile
  const int wn = (wave % C::WAVES_N) * C::WN;  // wave col offset inside the tile
  const int kbytes = K >> 1;

  const int kfull = kbytes / BKB;  // tiles entirely inside K
  const bool has_tail = (kbytes % BKB) != 0;

  // Global -> LDS copies of the full tiles go straight into LDS
  // (global_load_lds_dwordx4: lane l of a wave writes 16 bytes at
  // M0 + 16 l).  Wave w's copy i fills tile rows 8 rb .. 8 rb + 7,
  // rb = 8 i + w (A rows first, then B rows), so lane l owns row
  // 8 rb + l / 8 and LDS slot l % 8 of it; it fetches the global chunk
  // that the swizzle puts in that slot.  Rows past the matrix edge re-read
  // the last row (their results are never stored).
  constexpr int NW = C::WAVES_M * C::WAVES_N;
  static_assert(CPR == 8 && C::ROWS % (8 * NW) == 0 && CH == C::ROWS / (8 * NW),
                "copy mapping assumes 128-byte rows and whole 8-row blocks per wave");
  const uint8_t* src[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int rb = NW * i + wave;
    const int r = 8 * rb + (lane >> 3);
    const int c = (lane & 7) ^ lds_swz<8>(r);
    src[i] = (r < BM) ? a_q + int64_t(min(m0 + r, M - 1)) * lda + 16 * c
                      : b_q + int64_t(min(n0 + r - BM, N - 1)) * ldb + 16 * c;
  }
  const uint32_t lds0 = lds_address(&smem[0][0]);
  // copy full tile t (clamped to the last full tile) into stage st
#define QR_COPY(st, t)                                                                     \
  {                                                                                        \
    const int64_t kb0_ = int64_t(min((t), kfull - 1)) * BKB;                               \
    _Pragma("unroll") for (int i = 0; i < CH; ++i)                                         \
        lds_copy16(src[i] + kb0_, lds0 + uint32_t((st) * C::STAGE + (NW * i + wave) * 1024)); \
  }

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16i{};

  const int frow = lane & 31;   // row (A) / column (B) of the fragment
  const int fhalf = lane >> 5;  // which 16-byte chunk of a 32-byte K-pair
  constexpr int KP = BKB / 32;  // 64-wide K-pairs per tile
  static_assert(KP == 4, "the schedule below assumes four K-pairs per tile");

  // Packed fragments of one K-pair (16 bytes per block and lane), their
  // widened int8 form, and the MFMAs.  Two sets of each: the reads run two
  // K-pairs ahead of the MFMAs and the widening one K-pair ahead.
  uint4 ra0[FM], rb0[FN], ra1[FM], rb1[FN];
  v4i al0[FM], ah0[FM], bl0[FN], bh0[FN], al1[FM], ah1[FM], bl1[FN], bh1[FN];
#define QR_READ(n, st, kp)                                                                    \
  _Pragma("unroll") for (int i = 0; i < FM; ++i) ra##n[i] =                                  \
      ld16(smem[st] + lds_off<BKB>(wm + i * 32 + frow, 2 * (kp) + fhalf));                  \
  _Pragma("unroll") for (int j = 0; j < FN; ++j) rb##n[j] =                                  \
      ld16(smem[st] + BM * BKB + lds_off<BKB>(wn + j * 32 + frow, 2 * (kp) + fhalf))
#define QR_WIDEN(n)                                                                           \
  _Pragma("unroll") for (int i = 0; i < FM; ++i) widen(ra##n[i], al##n[i], ah##n[i]);        \
  _Pragma("unroll") for (int j = 0; j < FN; ++j) widen(rb##n[j], bl##n[j], bh##n[j])
// (all low halves first: the two MFMAs into one accumulator are FM * FN
// instructions apart, not back to back)
#define QR_MFMA(n)                                                                            \
  _Pragma("unroll") for (int i = 0; i < FM; ++i)                                              \
  _Pragma("unroll") for (int j = 0; j < FN; ++j)                                              \
    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(al##n[i], bl##n[j], acc[i][j], 0, 0, 0); \
  _Pragma("unroll") for (int i = 0; i < FM; ++i)                                              \
  _Pragma("unroll") for (int j = 0; j < FN; ++j)                                              \
    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ah##n[i], bh##n[j], acc[i][j], 0, 0, 0);
  // One pipeline step: LDS reads first, then each MFMA followed by a share
  // of the next K-pair's widening, so the VALU work runs in the MFMAs'
  // shadow instead of ahead of them.
#define QR_INTERLEAVE()                                                    \
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * (FM + FN), 0);          \
  _Pragma("unroll") for (int q = 0; q < 2 * FM * FN; ++q) {               \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    \
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);                    \
  }
#define QR_STEP(rd, cur, st, kp) \
  QR_READ(rd, st, kp);           \
  QR_WIDEN(rd == 0 ? 1 : 0);     \
  QR_MFMA(cur);                  \
  QR_INTERLEAVE()

  // Three LDS stages; tile kt lives in stage kt % 3.  Step g (K-pair
  // g = 4 kt + kp) reads K-pair g + 2 from LDS into register set g % 2,
  // widens K-pair g + 1 (read one step earlier) into the other widened set,
  // and runs the MFMAs of K-pair g.  Per tile one barrier, between kp1 and
  // kp2:
  //   kp0: copy tile kt+2 into stage (kt+2) % 3 (= the stage of tile kt-1,
  //        whose reads all finished before the previous barrier); step
  //   kp1: step (reads tile kt's last K-pair); wait until tile kt+1 has
  //        landed (its copies were issued one tile earlier; only tile kt+2's
  //        CH may still be in flight); barrier
  //   kp2, kp3: steps whose reads are tile kt+1's first two K-pairs
  // Copies past the last full tile repeat it into a stage nobody reads
  // again, and the reads that run past the end are harmless, so every
  // iteration has the same counts.
  if (kfull > 0) {
    QR_COPY(0, 0);
    QR_COPY(1, 1);
    wait_vmcnt<CH>();  // tile 0 landed
    __syncthreads();
    QR_READ(0, 0, 0);
    QR_READ(1, 0, 1);
    QR_WIDEN(0);
    int st = 0;  // stage of tile kt
    for (int kt = 0; kt < kfull; ++kt) {
      const int st1 = st == 2 ? 0 : st + 1, st2 = st1 == 2 ? 0 : st1 + 1;
      QR_COPY(st2, kt + 2);
      // kp0: read kp2 into set 0, widen kp1 (set 1), MFMAs kp0 (set 0)
      QR_READ(0, st, 2);
      QR_WIDEN(1);
      QR_MFMA(0);
      QR_INTERLEAVE();
      // kp1: read kp3 into set 1, widen kp2 (set 0), MFMAs kp1 (set 1)
      QR_READ(1, st, 3);
      QR_WIDEN(0);
      QR_MFMA(1);
      QR_INTERLEAVE();
      wait_vmcnt<CH>();  // tile kt+1 landed
      __syncthreads();
      // kp2: read tile kt+1 kp0 into set 0, widen kp3 (set 1), MFMAs kp2 (set 0)
      QR_READ(0, st1, 0);
      QR_WIDEN(1);
      QR_MFMA(0);
      QR_INTERLEAVE();
      // kp3: read tile kt+1 kp1 into set 1, widen tile kt+1 kp0 (set 0), MFMAs kp3 (set 1)
      QR_READ(1, st1, 1);
      QR_WIDEN(0);
      QR_MFMA(1);
      QR_INTERLEAVE();
      st = st1;
    }
    wait_vmcnt<0>();  // the trailing repeat copies, before any stage is rewritten
  }
#undef QR_COPY
  if (has_tail) {  // the partial tile at the end of K: chunks past K read as zero
    __syncthreads();
    const int lrow = tid / CPR, lchunk = tid % CPR;
    const int kb0 = kfull * BKB;
    const bool ok = kb0 + 16 * lchunk < kbytes;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int r = lrow + C::ROWS_PER_PASS * i;
      const uint8_t* p = (r < BM) ? a_q + int64_t(min(m0 + r, M - 1)) * lda
                                  : b_q + int64_t(min(n0 + r - BM, N - 1)) * ldb;
      const uint4 v = ok ? ld16(p + kb0 + 16 * lchunk) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(smem[0] + lds_off<BKB>(r, lchunk)) = v;
    }
    __syncthreads();
#pragma unroll
    for (int kp = 0; kp < KP; ++kp) {
      QR_READ(0, 0, kp);
      QR_WIDEN(0);
      QR_MFMA(0);
    }
  }
#undef QR_READ
#undef QR_WIDEN
#undef QR_MFMA
#undef QR_INTERLEAVE
#undef QR_STEP

  // --- epilogue: acc / 256 -> fp32 * scale_x * scale_w -> fp16 -----------
  // The accumulators go through LDS so that each lane ends up with 8
  // consecutive columns of one row: 16-byte output stores instead of 2-byte
  // ones.  32x32 block layout: lane holds column (lane & 31); register r
  // holds row 8 * (r / 4) + 4 * (lane / 32) + (r % 4).  Each wave owns a
  // [WM][WN] int32 staging tile.  The writes (32 consecutive words of a row
  // per half wave) are conflict-free.  On the read side the 8 lanes of a row
  // fetch every other 16-byte piece of it with one ds_read_b128, so lane
  // (cg, r0) takes the half (cg ^ r0) & 1 of its 8 columns first: the pieces
  // of rows r0 and r0 + 1 then interleave.  SQ_LDS_BANK_CONFLICT on a probe
  // of this read pattern: none, against 8 cycles per read with the earlier
  // [WN + 8] rows and fixed order (the kernel's whole 262,144 per launch).
  constexpr int WM = C::WM, WN = C::WN, LDS_ROW = WN;
  static_assert(C::WAVES_M * C::WAVES_N * WM * LDS_ROW * 4 <= 3 * C::STAGE,
                "staging tiles must fit in the pipeline's LDS");
  __syncthreads();  // every wave is done reading the last K tile
  int32_t* stg = reinterpret_cast<int32_t*>(&smem[0][0]) + wave * (WM * LDS_ROW);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        stg[row * LDS_ROW + j * 32 + (lane & 31)] = acc[i][j][r] >> 8;
      }
  __syncthreads();
  // lane -> columns 8 cg .. 8 cg + 7 of the wave tile, rows lane / 8 + 8 s
  constexpr int CG = WN / 8, RSTEP = 64 / CG;
  static_assert(CG == 8 && RSTEP % 2 == 0, "the read order below pairs rows r0 and r0 + 1");
  const int cg = lane % CG, r0 = lane / CG;
  const int first = (cg ^ r0) & 1;  // half of the 8 columns read first
  const int col0 = n0 + wn + 8 * cg;
  float sw[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) sw[k] = __half2float(b_scale[min(col0 + k, N - 1)]);
  const bool full_cols = col0 + 8 <= N;
  const bool vec_c = full_cols && (ldc % 8) == 0 && (reinterpret_cast<uintptr_t>(c) % 16) == 0;
  const bool vec_acc = full_cols && acc_out && (ld_acc % 4) == 0 &&
                       (reinterpret_cast<uintptr_t>(acc_out) % 16) == 0;
#pragma unroll
  for (int sidx = 0; sidx < WM / RSTEP; ++sidx) {
    const int lrow_ = r0 + RSTEP * sidx;
    const int row = m0 + wm + lrow_;
    if (row >= M) continue;
    const float sx = __half2float(a_scale[row]);
    const int4 u0 = *reinterpret_cast<const int4*>(stg + lrow_ * LDS_ROW + 8 * cg + 4 * first);
    const int4 u1 =
        *reinterpret_cast<const int4*>(stg + lrow_ * LDS_ROW + 8 * cg + 4 * (1 - first));
    const int4 v0 = first ? u1 : u0, v1 = first ? u0 : u1;
    const int v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    __half h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = __float2half_rn((float(v[k]) * sx) * sw[k]);
    __half* crow = c + int64_t(row) * ldc + col0;
    if (vec_c) {
      uint4 pk;
      __builtin_memcpy(&pk, h, 16);
      *reinterpret_cast<uint4*>(crow) = pk;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (col0 + k < N) crow[k] = h[k];
    }
    if (acc_out) {
      int32_t* arow = acc_out + int64_t(row) * ld_acc + col0;
      if (vec_acc) {
        *reinterpret_cast<int4*>(arow) = v0;
        *reinterpret_cast<int4*>(arow + 4) = v1;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (col0 + k < N) arow[k] = v[k];
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
  if (total * C::THREADS > 0xffffffffLL) {  // work items of one grid dimension
    set_error("too many tiles");
    return QUAROT_ERR_UNSUPPORTED;
  }
  hipLaunchKernelGGL(w4a4_gemm_kernel<C>, dim3(unsigned(total)), dim3(C::THREADS), 0, stream,
                     a_q, lda, a_scale, b_q, ldb, b_scale, int(M), int(N), int(K), c, ldc,
                     acc_out, ld_acc, tiles_m, tiles_n);
  return check_launch("w4a4_gemm");
}

// ---------------------------------------------------------------------------
// Large-tile variant for problems with many output tiles: four waves (one
// per SIMD), each owning a 128 x 128 block of the output (4 x 4 MFMA blocks,
// 256 accumulator registers).  Against 64 x 64 wave tiles this halves the
// LDS bytes and the widening instructions per MFMA; both cost clock under
// the chip's power limit as well as issue cycles.  K tiles are 128 codes
// (64 bytes per row, two K-pairs) in a ring of four LDS stages: the copy of
// tile kt + 3 is issued while tile kt is computed, so each copy has two
// tiles of compute to land.
template <int WAVES_M_, int WAVES_N_, int WM_, int WN_, int NST_>
struct BigCfg {
  static constexpr int BKB = 64, CPR = 4, NST = NST_, KP = 2;
  static_assert(NST >= 3, "the ring needs a stage being computed, one landed and one in flight");
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, NW = WAVES_M * WAVES_N;
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int BM = WAVES_M * WM, BN = WAVES_N * WN;
  static constexpr int THREADS = 64 * NW;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int ROWS = BM + BN;
  static constexpr int STAGE = ROWS * BKB;
  static constexpr int BLK = ROWS / 16;   // 16-row (1 KiB) blocks per tile
  static constexpr int CH = BLK / NW;     // copy instructions per wave per tile
  static_assert(BLK % NW == 0 && BM % 16 == 0, "copy blocks must split evenly and not straddle A/B");
};

using BigCfg4 = BigCfg<2, 2, 128, 128, 4>;  // 256 x 256 workgroup tile

template <class C>
__global__ __launch_bounds__(C::THREADS) void w4a4_gemm_big_kernel(
    const uint8_t* __restrict__ a_q, int64_t lda, const __half* __restrict__ a_scale,
    const uint8_t* __restrict__ b_q, int64_t ldb, const __half* __restrict__ b_scale,
    int M, int N, int K, __half* __restrict__ c, int64_t ldc, int32_t* __restrict__ acc_out,
    int64_t ld_acc, int tiles_m, int tiles_n) {
  constexpr int FM = C::FM, FN = C::FN, CH = C::CH, BM = C::BM, BN = C::BN;
  constexpr int BKB = C::BKB, NST = C::NST, NW = C::NW;
  __shared__ __attribute__((aligned(16))) uint8_t smem[NST * C::STAGE];

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave / C::WAVES_N) * C::WM;
  const int wn = (wave % C::WAVES_N) * C::WN;
  const int kbytes = K >> 1;
  const int kfull = kbytes / BKB;
  const bool has_tail = (kbytes % BKB) != 0;

  // Copy i of wave w fills tile rows 16 b .. 16 b + 15, b = NW i + w (A rows,
  // then B rows): lane l owns row 16 b + l / 4 and LDS slot l % 4 of it, and
  // fetches the global chunk the swizzle puts in that slot.  Rows past the
  // matrix edge re-read the last row (their results are never stored).
  const uint8_t* src[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int r = 16 * (NW * i + wave) + (lane >> 2);
    const int ch = (lane & 3) ^ lds_swz<4>(r);
    src[i] = (r < BM) ? a_q + int64_t(min(m0 + r, M - 1)) * lda + 16 * ch
                      : b_q + int64_t(min(n0 + r - BM, N - 1)) * ldb + 16 * ch;
  }
  const uint32_t lds0 = lds_address(&smem[0]);
#define QB_COPY(st, t)                                                                     \
  {                                                                                        \
    const int64_t kb0_ = int64_t(min((t), kfull - 1)) * BKB;                               \
    _Pragma("unroll") for (int i = 0; i < CH; ++i)                                         \
        lds_copy16(src[i] + kb0_, lds0 + uint32_t((st) * C::STAGE + (NW * i + wave) * 1024)); \
  }

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16i{};

  const int frow = lane & 31;
  const int fhalf = lane >> 5;

  uint4 ra0[FM], rb0[FN], ra1[FM], rb1[FN];
  v4i al0[FM], ah0[FM], bl0[FN], bh0[FN], al1[FM], ah1[FM], bl1[FN], bh1[FN];
#define QB_READ(n, st, kp)                                                                    \
  _Pragma("unroll") for (int i = 0; i < FM; ++i) ra##n[i] =                                  \
      ld16(smem + (st) * C::STAGE + lds_off<BKB>(wm + i * 32 + frow, 2 * (kp) + fhalf));    \
  _Pragma("unroll") for (int j = 0; j < FN; ++j) rb##n[j] =                                  \
      ld16(smem + (st) * C::STAGE + BM * BKB + lds_off<BKB>(wn + j * 32 + frow, 2 * (kp) + fhalf))
#define QB_WIDEN(n)                                                                           \
  _Pragma("unroll") for (int i = 0; i < FM; ++i) widen(ra##n[i], al##n[i], ah##n[i]);        \
  _Pragma("unroll") for (int j = 0; j < FN; ++j) widen(rb##n[j], bl##n[j], bh##n[j])
#define QB_MFMA(n)                                                                            \
  _Pragma("unroll") for (int i = 0; i < FM; ++i)                                              \
  _Pragma("unroll") for (int j = 0; j < FN; ++j)                                              \
    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(al##n[i], bl##n[j], acc[i][j], 0, 0, 0); \
  _Pragma("unroll") for (int i = 0; i < FM; ++i)                                              \
  _Pragma("unroll") for (int j = 0; j < FN; ++j)                                              \
    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ah##n[i], bh##n[j], acc[i][j], 0, 0, 0);

  // One step in 2 FM groups, each fenced off for the scheduler: group g runs
  // the MFMAs of accumulator row g % FM (the low halves first, then the
  // high halves), and the FM + FN raw fragments are spread over the groups
  // (fragment f in group f * 2 FM / (FM + FN)): each is read for K-pair
  // g + 2 into raw set RD and widened from raw set WD.  In the first step
  // of a tile the CH copies of the next tile are spread the same way.  The
  // global-to-LDS copies and LDS reads thereby sit between MFMAs instead of
  // stalling the wave that issues them in a burst.
  constexpr int NG = 2 * FM, NF = FM + FN;
#define QB_GSTEP(RD, WD, ST, KP, DO_COPY)                                                          \
  _Pragma("unroll") for (int g = 0; g < NG; ++g) {                                               \
    _Pragma("unroll") for (int f = 0; f < NF; ++f) {                                             \
      if (f * NG / NF != g) continue;                                                             \
      if (f < FM)                                                                                 \
        ra##RD[f] = ld16(smem + (ST) * C::STAGE + lds_off<BKB>(wm + f * 32 + frow, 2 * (KP) + fhalf)); \
      else                                                                                        \
        rb##RD[f - FM] = ld16(smem + (ST) * C::STAGE + BM * BKB +                                 \
                              lds_off<BKB>(wn + (f - FM) * 32 + frow, 2 * (KP) + fhalf));         \
    }                                                                                             \
    if (g < FM) {                                                                                 \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) acc[g][j] =                                  \
          __builtin_amdgcn_mfma_i32_32x32x32_i8(al##RD[g], bl##RD[j], acc[g][j], 0, 0, 0);        \
    } else {                                                                                      \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) acc[g - FM][j] =                             \
          __builtin_amdgcn_mfma_i32_32x32x32_i8(ah##RD[g - FM], bh##RD[j], acc[g - FM][j], 0, 0, 0); \
    }                                                                                             \
    _Pragma("unroll") for (int f = 0; f < NF; ++f) {                                             \
      if (f * NG / NF != g) continue;                                                             \
      if (f < FM) widen(ra##WD[f], al##WD[f], ah##WD[f]);                                        \
      else widen(rb##WD[f - FM], bl##WD[f - FM], bh##WD[f - FM]);                                \
    }                                                                                             \
    if (DO_COPY) {                                                                                \
      _Pragma("unroll") for (int cc = 0; cc < CH; ++cc) {                                        \
        if (cc * NG / CH != g) continue;                                                          \
        lds_copy16(src[cc] + kbc, lds0 + uint32_t(stc * C::STAGE + (NW * cc + wave) * 1024));     \
      }                                                                                           \
    }                                                                                             \
    _Pragma("unroll") for (int q = 0; q < FN; ++q) {                                              \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         \
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);                                         \
    }                                                                                             \
    __builtin_amdgcn_sched_barrier(0);                                                           \
  }

  // K-pair g = 2 kt + kp.  Step g reads K-pair g + 2 (tile kt + 1, same kp)
  // into register set g % 2, widens K-pair g + 1 into the other widened set
  // and runs the MFMAs of K-pair g.  Iteration kt starts by waiting until
  // tile kt + 1 has landed (its copy was issued NST - 2 iterations earlier;
  // only the copies of tiles kt + 2 .. kt + NST - 2 may still be in flight)
  // and a barrier, after which every wave has consumed tile kt - 1, so its
  // stage takes the copy of tile kt + NST - 1.  Copies past the last full
  // tile repeat it into stages that are never read as real data.
  if (kfull > 0) {
#pragma unroll
    for (int t = 0; t < NST - 1; ++t) QB_COPY(t, t);
    wait_vmcnt<(NST - 2) * CH>();  // tile 0 landed
    __syncthreads();
    QB_READ(0, 0, 0);
    QB_READ(1, 0, 1);
    QB_WIDEN(0);
    int st1 = 1 % NST, stc = NST - 1;  // stages of tiles kt + 1 and kt + NST - 1
    for (int kt = 0; kt < kfull; ++kt) {
      wait_vmcnt<(NST - 3) * CH>();  // tile kt + 1 landed
      __syncthreads();
      {
        const int64_t kbc = int64_t(min(kt + NST - 1, kfull - 1)) * BKB;
        // kp0: read tile kt+1 kp0 into set 0, widen tile kt kp1 (set 1), MFMAs tile kt kp0 (set 0)
        QB_GSTEP(0, 1, st1, 0, true);
        // kp1: read tile kt+1 kp1 into set 1, widen tile kt+1 kp0 (set 0), MFMAs tile kt kp1 (set 1)
        QB_GSTEP(1, 0, st1, 1, false);
      }
      st1 = st1 == NST - 1 ? 0 : st1 + 1;
      stc = stc == NST - 1 ? 0 : stc + 1;
    }
    wait_vmcnt<0>();
  }
#undef QB_COPY
  if (has_tail) {  // the partial tile at the end of K: chunks past K read as zero
    __syncthreads();
    const int kb0 = kfull * BKB;
    for (int idx = tid; idx < C::ROWS * C::CPR; idx += C::THREADS) {
      const int r = idx / C::CPR, lchunk = idx % C::CPR;
      const uint8_t* p = (r < BM) ? a_q + int64_t(min(m0 + r, M - 1)) * lda
                                  : b_q + int64_t(min(n0 + r - BM, N - 1)) * ldb;
      const bool ok = kb0 + 16 * lchunk < kbytes;
      const uint4 v = ok ? ld16(p + kb0 + 16 * lchunk) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(smem + lds_off<BKB>(r, lchunk)) = v;
    }
    __syncthreads();
#pragma unroll
    for (int kp = 0; kp < C::KP; ++kp) {
      QB_READ(0, 0, kp);
      QB_WIDEN(0);
      QB_MFMA(0);
    }
  }
#undef QB_READ
#undef QB_WIDEN
#undef QB_MFMA
#undef QB_GSTEP

  // --- epilogue: acc / 256 -> fp32 * scale_x * scale_w -> fp16 -----------
  // One 32-row block of the wave tile at a time goes through a per-wave
  // [32][WN + 8] int32 staging tile, so each lane then owns 8 consecutive
  // columns of a row (16-byte output stores).
  constexpr int WN = C::WN, LDS_ROW = WN + 8;
  static_assert(NW * 32 * LDS_ROW * 4 <= NST * C::STAGE, "staging tiles must fit");
  constexpr int CG = WN / 8, RSTEP = 64 / CG;
  const int cg = lane % CG, r0 = lane / CG;
  const int col0 = n0 + wn + 8 * cg;
  float sw[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) sw[k] = __half2float(b_scale[min(col0 + k, N - 1)]);
  const bool full_cols = col0 + 8 <= N;
  const bool vec_c = full_cols && (ldc % 8) == 0 && (reinterpret_cast<uintptr_t>(c) % 16) == 0;
  const bool vec_acc = full_cols && acc_out && (ld_acc % 4) == 0 &&
                       (reinterpret_cast<uintptr_t>(acc_out) % 16) == 0;
  int32_t* stg = reinterpret_cast<int32_t*>(smem) + wave * (32 * LDS_ROW);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    __syncthreads();  // the K loop's reads (first block) or the previous block's reads are done
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        stg[row * LDS_ROW + j * 32 + (lane & 31)] = acc[i][j][r] >> 8;
      }
    __syncthreads();
#pragma unroll
    for (int sidx = 0; sidx < 32 / RSTEP; ++sidx) {
      const int lrow_ = r0 + RSTEP * sidx;
      const int row = m0 + wm + 32 * i + lrow_;
      if (row >= M) continue;
      const float sx = __half2float(a_scale[row]);
      const int4 v0 = *reinterpret_cast<const int4*>(stg + lrow_ * LDS_ROW + 8 * cg);
      const int4 v1 = *reinterpret_cast<const int4*>(stg + lrow_ * LDS_ROW + 8 * cg + 4);
      const int v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      __half h[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) h[k] = __float2half_rn((float(v[k]) * sx) * sw[k]);
      __half* crow = c + int64_t(row) * ldc + col0;
      if (vec_c) {
        uint4 pk;
        __builtin_memcpy(&pk, h, 16);
        *reinterpret_cast<uint4*>(crow) = pk;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (col0 + k < N) crow[k] = h[k];
      }
      if (acc_out) {
        int32_t* arow = acc_out + int64_t(row) * ld_acc + col0;
        if (vec_acc) {
          *reinterpret_cast<int4*>(arow) = v0;
          *reinterpret_cast<int4*>(arow + 4) = v1;
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (col0 + k < N) arow[k] = v[k];
        }
      }
    }
  }
}

template <class C>
int launch_big(const uint8_t* a_q, int64_t lda, const __half* a_scale, const uint8_t* b_q,
               int64_t ldb, const __half* b_scale, int64_t M, int64_t N, int64_t K, __half* c,
               int64_t ldc, int32_t* acc_out, int64_t ld_acc, hipStream_t stream) {
  const int tiles_m = int((M + C::BM - 1) / C::BM);
  const int tiles_n = int((N + C::BN - 1) / C::BN);
  const int64_t total = int64_t(tiles_m) * tiles_n;
  if (total * C::THREADS > 0xffffffffLL) {  // work items of one grid dimension
    set_error("too many tiles");
    return QUAROT_ERR_UNSUPPORTED;
  }
  hipLaunchKernelGGL(w4a4_gemm_big_kernel<C>, dim3(unsigned(total)), dim3(C::THREADS), 0, stream,
                     a_q, lda, a_scale, b_q, ldb, b_scale, int(M), int(N), int(K), c, ldc,
                     acc_out, ld_acc, tiles_m, tiles_n);
  return check_launch("w4a4_gemm");
}

}  // namespace

int launch_w4a4_gemm(const uint8_t* a_q, int64_t lda, const __half* a_scale,
                     const uint8_t* b_q, int64_t ldb, const __half* b_scale,
                     int64_t M, int64_t N, int64_t K, __half* c, int64_t ldc,
                     int32_t* acc_out, int64_t ld_acc, hipStream_t stream) {
  // 256 x 256 tiles when they alone fill every CU; otherwise 128 x 256 tiles
  // (e.g. 2048 x 4096 outputs are 128 large tiles but 256 of the smaller).
  const int64_t big_tiles = ((M + BigCfg4::BM - 1) / BigCfg4::BM) * ((N + BigCfg4::BN - 1) / BigCfg4::BN);
  if (big_tiles >= 256)
    return launch_big<BigCfg4>(a_q, lda, a_scale, b_q, ldb, b_scale, M, N, K, c, ldc, acc_out,
                               ld_acc, stream);
  return launch_cfg<Cfg8>(a_q, lda, a_scale, b_q, ldb, b_scale, M, N, K, c, ldc, acc_out,
                          ld_acc, stream);
}

}  // namespace quarot
