// Rotate+quant of plain rows of d = 512 m (H_512 (x) H_m; d = 12288 runs as
// 512 groups of 24 under H_2 (x) H_12) with every butterfly stage in
// registers.  One 256-thread workgroup owns one row, two per CU.  H_m is the
// caller's matrix, handed in as bit masks.  With SWIGLU the row is the gated
// FFN product c = SiLU(gate) * up (section 3.4 Stage 1b of the same page),
// formed in fp32 on compact 16-byte chunks and split as in had_quant_kron:
// hi = fp16(c), lo = fp16((c - hi) 2^11), staged in the wave's own slice of
// the LDS row area and fed to the matrix cores against H_m and 2^-11 H_m.
// The d = 28672 rows keep had_quant_kron: there (1024 groups) phase 2 would
// take five stages over 32 groups with one-byte code units, which measured
// 3-4% slower than the DPP butterflies it saves (77-81 against 74-77 us).
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary), section 3.4 Stage 1a: for d = 2^n m the Hadamard is
// H_{2^n} (x) H_m with a known H_m, computable in O(d (m + n)); Stage 1b:
// the online Hadamard before the down-projection.
//
// Element e = a * m + b, a = 0..NP-1 (the power-of-two index, bits a0 ..),
// b = 0..m-1.  The DPP butterflies of a lane-major layout cost about twice a
// register butterfly on this chip (a v_fmac_f32_dpp issues at about half the
// rate of a v_fmac_f32), so the layout keeps every stage in registers:
//   phase 1  wave w, lane l = n + 16 g, tile t (of 8) load the 16-byte chunk
//            b = 8 g .. 8 g + 7 of group a = 128 w + 16 t + n, as now the A
//            operand of v_mfma_f32_16x16x32_f16; H_m (rows 0-15 and 16-31)
//            is the B operand.  D = X^T H_m^T then holds, in lane n + 16 g,
//            b' = n (and 16 + n) of the four groups 128 w + 16 t + 4 g + i,
//            i = 0..3 in its registers.  Butterflies over a0, a1 (i) and
//            a4, a5, a6 (t), all in registers; the row goes to LDS b-major
//            (row b', group a), four consecutive groups per 16-byte store.
//   phase 2  task (c, u): c fixes a0, a1, a4, a5, a6 (32 combos), u a run
//            of four consecutive b.  It reads its four values of each of the
//            16 groups that differ in a2, a3, a7, a8, runs those stages in
//            registers, joins the workgroup maximum, quantises and writes
//            16-bit code units to LDS; the row's codes then leave in 16-byte
//            stores.
#pragma once

#include "kron_rows.h"

namespace quarot {

template <int M, int NP>
struct KronTCfg {
  static constexpr int D = NP * M;
  static constexpr int AW = 128;  // groups per wave in phase 1
  static constexpr int TILES = AW / 16;
  static constexpr int NWAVE = NP / AW;
  static constexpr int THREADS = 64 * NWAVE;
  static constexpr int BLOCKS_PER_CU = NWAVE == 4 ? 2 : 1;
  static constexpr int QN = NP / 32;  // phase-2 groups: a2, a3, a7, a8
  static constexpr int BW = 64 / QN;  // b per task: 4
  static constexpr int UNITS = M / BW;
  static constexpr int TASKS = 32 * UNITS;
  static constexpr int HALVES = (M > 16) ? 2 : 1;
  // LDS row of one b: the NP groups plus a pad of four floats.  Group a of
  // a row sits at column a ^ kront_swz(a) (bits 2, 3 XOR a5, a6).  4-byte
  // LDS accesses go through 32 banks, half a wave per cycle; the phase-2
  // reads of a half wave (32 combos: a0, a1, a4, a5, a6) then hit 32
  // distinct banks, and the phase-1 16-byte writes stay conflict-free with
  // this pad (SQ_LDS_BANK_CONFLICT on a probe of both patterns: none).
  static constexpr int AP = NP + 4;
  static constexpr int CODE_OFF = M * AP;  // the codes follow the fp32 row
  // Code area: the row's D / 32 16-byte chunks with one chunk of pad after
  // every CODE_BLK.  A half wave's 16-bit code writes (32 combos, a stride
  // of M / 4 units) step by multiples of 32 dwords over a5 and a6, so at
  // m = 24 they would share 8 banks; the pad moves each 96-dword block by 4
  // banks, and a model of every (unit, q) write then finds 32 distinct
  // banks.
  static constexpr int CODE_CHUNKS = D / 32;
  static constexpr int CODE_BLK = 24;
  static constexpr int QSTEP = (M / BW) * 128;  // code units between q and q + 4
  static constexpr int LDS_BYTES =
      CODE_OFF * 4 + 16 * (CODE_CHUNKS + (CODE_CHUNKS + CODE_BLK - 1) / CODE_BLK);
  static_assert(M == 24, "the code-area pad is laid out for m = 24");
  static_assert(QSTEP % (8 * CODE_BLK) == 0, "q + 4 keeps a unit's place in its pad block");
  static_assert(NP == 512, "four waves per row");
  static_assert(TASKS <= THREADS && TASKS % 64 == 0, "whole waves of phase-2 tasks");
};

// column offset of group a within its LDS row: a ^ kront_swz(a)
__device__ __forceinline__ constexpr int kront_swz(int a) {
  return (((a >> 5) & 1) << 2) | (((a >> 6) & 1) << 3);
}

// SWIGLU: x is the gate projection and up the up projection; the row is
// SiLU(x) * up.  Otherwise up is unused and the row is x.
template <int M, bool CLAMP, int NP, bool SWIGLU>
__global__ __launch_bounds__((KronTCfg<M, NP>::THREADS), 2) void had_quant_kront(
    const __half* __restrict__ x, int64_t ld_x, const __half* __restrict__ up, int64_t ld_up,
    int64_t rows, const int8_t* __restrict__ signs, HadMasks hm, float clip_ratio,
    uint8_t* __restrict__ q_out, int64_t ld_q, __half* __restrict__ scale_out,
    float* __restrict__ x_rot, float norm) {
  using C = KronTCfg<M, NP>;
  extern __shared__ float4 kront_lds[];  // the row in fp32 (b-major), then its codes
  float* buf = reinterpret_cast<float*>(kront_lds);
  __shared__ float red[C::NWAVE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  constexpr int TILES = C::TILES, AW = C::AW, AP = C::AP, BW = C::BW, QN = C::QN;

  // valid elements of this lane's chunk: b = 8 g .. 8 g + cnt - 1 (cnt 8 or
  // 0 for m = 24; 8 or 4 for m = 28).  The lane loads 16 bytes inside its
  // group: a full chunk at b = 8 g, a half chunk (the group's last four) at
  // b = 8 g - 4 so the wanted values sit in the upper half, lanes past m at
  // the group start.  Unwanted slots meet zero rows of the B operand.
  const int cnt = min(8, max(0, M - 8 * g));
  const int off16 = cnt == 8 ? 8 * g : (cnt == 4 ? 8 * g - 4 : 0);
  // B operands: B[k][b'] = H_m[b'][k] for b' = n (and 16 + n), k = the
  // lane's K slots, zero padded: slot j pairs with column 8 g + j, or
  // 8 g + j - 4 for a half chunk.  (The same registers as the A operand of
  // the lane-major layout: the two operands share one lane layout.)
  const int shift = cnt == 4 ? 4 : 0;
  const uint32_t nz_lo = mask_row(hm.nz, n) >> (8 * g), neg_lo = mask_row(hm.neg, n) >> (8 * g);
  const uint32_t nz_hi = mask_row(hm.nz, n + 16) >> (8 * g);
  const uint32_t neg_hi = mask_row(hm.neg, n + 16) >> (8 * g);
  half8_t h_lo, h_hi, hs_lo, hs_hi;  // hs: H_m 2^-11 for the gated product's low parts
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool in = j >= shift;
    h_lo[j] = in ? had_entry(nz_lo, neg_lo, j - shift) : _Float16(0.0f);
    h_hi[j] = in ? had_entry(nz_hi, neg_hi, j - shift) : _Float16(0.0f);
    hs_lo[j] = h_lo[j] * _Float16(1.0f / 2048.0f);
    hs_hi[j] = h_hi[j] * _Float16(1.0f / 2048.0f);
  }
  // The gated product is formed on a compact layout: the wave's AW groups
  // (contiguous in the row) are J 16-byte chunks per lane and stream, every
  // element real.  Its fp16 sign-bit masks are XORed into up.
  constexpr int J = AW * M / 512;
  static_assert(!SWIGLU || AW * M % 512 == 0, "whole compact chunks per lane");
  uint4 cmask[SWIGLU ? J : 1];
  if constexpr (SWIGLU) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      uint32_t w0 = 0, w1 = 0;
      if (signs) {
        const int e = AW * wave * M + 512 * j + 8 * lane;
        __builtin_memcpy(&w0, signs + e, 4);
        __builtin_memcpy(&w1, signs + e + 4, 4);
      }
      cmask[j] = sign_masks8(w0, w1);
    }
  }
  // signs of this lane's phase-1 elements (the same for every row), as fp16
  // sign-bit masks: group a = 128 wave + 16 t + n
  uint4 mask[SWIGLU ? 1 : TILES];
#pragma unroll
  for (int t = 0; t < (SWIGLU ? 0 : TILES); ++t) {
    uint32_t w0 = 0, w1 = 0;
    if (signs) {
      const int a = AW * wave + 16 * t + n;
      __builtin_memcpy(&w0, signs + a * M + off16, 4);
      __builtin_memcpy(&w1, signs + a * M + off16 + 4, 4);
    }
    mask[t] = sign_masks8(w0, w1);
  }

  // phase-2 task of this thread: combo c (a0, a1 = c bits 0, 1; a4, a5, a6 =
  // c bits 2-4), run u of BW b.  A wave takes units 2 w and 2 w + 1 of all
  // 32 combos.
  const bool task_on = tid < C::TASKS;
  const int combo = tid & 31, unit = tid >> 5;
  const int abase = (combo & 3) + ((combo >> 2) << 4);

  // one row's loads: tiles of 16 groups, or (gated) J compact chunks of both
  // inputs as buffer loads (one 32-bit lane offset for every chunk)
  constexpr int NR = SWIGLU ? J : TILES, TU = SWIGLU ? J : 1;
  const int lane_off = 2 * (AW * wave * M + 8 * lane);
  auto load_chunk = [&](int64_t row, int j, uint4& r, uint4& ru) {
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__half*>(x + row * ld_x), 0, 2 * C::D, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__half*>(up + row * ld_up), 0, 2 * C::D, 0x00020000);
    r = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, lane_off + 1024 * j, 0, 0));
    ru = __builtin_bit_cast(uint4,
                            __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off + 1024 * j, 0, 0));
  };
  auto load_row = [&](int64_t row, uint4 (&raw)[NR], uint4 (&raw_u)[TU]) {
    if constexpr (SWIGLU) {
#pragma unroll
      for (int j = 0; j < J; ++j) load_chunk(row, j, raw[j], raw_u[j]);
    } else {
      const __half* src = x + row * ld_x;
#pragma unroll
      for (int t = 0; t < TILES; ++t)
        __builtin_memcpy(&raw[t], src + (AW * wave + 16 * t + n) * M + off16, 16);
    }
  };
  // Gated product staging: float f (< 24 AW) of the wave's staging area lives
  // in the wave's own slice of the b-major row area (rows of AW floats at
  // column AW wave), which only this wave writes in write_row, after it has
  // read the staged parts back.  hi parts take floats 0 .. AW M / 2 - 1, lo
  // parts the rest (AW M floats in all: the slice's M rows).
  static_assert(!SWIGLU || M == 24, "the staging area is the wave's 24 rows of AW floats");
  auto stage = [&](int f) -> float* { return buf + (f >> 7) * AP + AW * wave + (f & 127); };

  // ---- phase 1: H_m on the matrix cores (D = X^T H_m^T), then the
  // butterflies over a0, a1 (register bits 0, 1) and a4-a6 (bits 3-5) ------
  // register r = 8 t + 4 h + i: b' = 16 h + n of group 128 w + 16 t + 4 g + i
  // (gated product: nrow < rows issues the next row's loads chunk by chunk
  // as soon as each chunk's registers are free, so they overlap the product
  // phase instead of following it)
  auto phase1 = [&](uint4 (&raw)[NR], uint4 (&raw_u)[TU], float (&v)[8 * TILES],
                    int64_t nrow) {
    constexpr int kLo = AW * M / 2;  // float offset of the lo parts (after AW M / 2 of hi)
    if constexpr (SWIGLU) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint4 um = make_uint4(raw_u[j].x ^ cmask[j].x, raw_u[j].y ^ cmask[j].y,
                                    raw_u[j].z ^ cmask[j].z, raw_u[j].w ^ cmask[j].w);
        uint4 hi, lo;
        swiglu_split8(raw[j], um, hi, lo);
        if (nrow < rows) load_chunk(nrow, j, raw[j], raw_u[j]);
        *reinterpret_cast<uint4*>(stage(256 * j + 4 * lane)) = hi;
        *reinterpret_cast<uint4*>(stage(kLo + 256 * j + 4 * lane)) = lo;
      }
      // the wave reads back what its own lanes wrote: LDS completes a wave's
      // accesses in order once they have all been issued and counted
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
      float4_t d0, d1;
      if constexpr (SWIGLU) {
        // chunk b = 8 g .. 8 g + 7 of group 16 t + n (lanes past m read the
        // group's first chunk, against zero rows of H): element e = (16 t +
        // n) m + 8 g is float e / 2 of the staged parts
        const int f = ((16 * t + n) * M + (cnt > 0 ? 8 * g : 0)) >> 1;
        const half8_t ah = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4*>(stage(f)));
        const half8_t al =
            __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4*>(stage(kLo + f)));
        // X hi against H_m, then X lo against 2^-11 H_m onto it (exact products)
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, h_lo, zero, 0, 0, 0);
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, hs_lo, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, h_hi, zero, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, hs_hi, d1, 0, 0, 0);
      } else {
        const uint4 r = make_uint4(raw[t].x ^ mask[t].x, raw[t].y ^ mask[t].y,
                                   raw[t].z ^ mask[t].z, raw[t].w ^ mask[t].w);
        const half8_t aop = __builtin_bit_cast(half8_t, r);
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, h_lo, zero, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, h_hi, zero, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[8 * t + q] = d0[q];
        v[8 * t + 4 + q] = d1[q];
      }
    }
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
      if (h == 4) continue;  // register bit 2 is the MFMA half (b')
#pragma unroll
      for (int r = 0; r < 8 * TILES; ++r)
        if ((r & h) == 0) {
          const float a = v[r], b = v[r + h];
          v[r] = a + b;
          v[r + h] = a - b;
        }
    }
  };
  // to LDS, b-major: element (a, b') at b' AP + (a ^ kront_swz(a)); four
  // consecutive groups per store (a5, a6 are bits 1, 2 of t, so the swizzle
  // of a tile is a constant XOR on the lane's 4 g)
  auto write_row = [&](const float (&v)[8 * TILES]) {
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int h = 0; h < C::HALVES; ++h) {
        const int bp = 16 * h + n;
        if (bp < M)
          *reinterpret_cast<float4*>(buf + bp * AP + AW * wave + 16 * t +
                                     ((4 * g) ^ kront_swz(16 * t))) =
              make_float4(v[8 * t + 4 * h], v[8 * t + 4 * h + 1], v[8 * t + 4 * h + 2],
                          v[8 * t + 4 * h + 3]);
      }
  };
  // ---- phase 2: a2, a3 and the group bits from a7 up, in registers ------
  // register BW q + k holds b = BW unit + k of group a(q) = abase +
  // 4 (q & 3) + 128 (q >> 2).  Returns the task's largest |value|.
  constexpr int NV = QN * BW;
  auto phase2 = [&](float (&v)[NV]) -> float {
    float amax = 0.0f;
    if (task_on) {
      // column of a(q) = abase + ((4 (q & 3)) ^ swz) + 128 (q >> 2): the
      // swizzle comes from abase's a5, a6 only
      const int swz = kront_swz(abase);
      const float* src = buf + BW * unit * AP + abase;
      int col[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) col[j] = (4 * j) ^ swz;
#pragma unroll
      for (int k = 0; k < BW; ++k)
#pragma unroll
        for (int q = 0; q < QN; ++q)
          v[BW * q + k] = src[k * AP + col[q & 3] + 128 * (q >> 2)];
#pragma unroll
      for (int h = 1; h < QN; h <<= 1)
#pragma unroll
        for (int q = 0; q < QN; ++q)
          if ((q & h) == 0)
#pragma unroll
            for (int k = 0; k < BW; ++k) {
              const float a = v[BW * q + k], b = v[BW * (q + h) + k];
              v[BW * q + k] = a + b;
              v[BW * (q + h) + k] = a - b;
            }
#pragma unroll
      for (int r = 0; r < NV; ++r) amax = fmaxf(amax, fabsf(v[r]));
    }
    return amax;
  };
  // the row's scale from the per-wave maxima, then its codes to the LDS code
  // area (four codes per 16-bit unit) and the optional fp32 copy.  Group
  // a(q)'s run starts at element a(q) M + 4 unit: code unit a(q) (M / 4) +
  // unit, placed past the pad chunks before it.
  auto quantize = [&](const float (&v)[NV], int64_t row) -> __half {
    float amax = red[0];
#pragma unroll
    for (int w = 1; w < C::NWAVE; ++w) amax = fmaxf(amax, red[w]);
    const __half s16 = row_scale_fp16(amax * norm, clip_ratio);
    const float kq = inv_scale(s16) * norm;
    if (task_on) {
      // unit index u lives at u + 8 (u / (8 CODE_BLK)): 8 units a chunk
      int cpad[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = abase * (M / BW) + unit + (M / BW) * 4 * j;
        cpad[j] = c + 8 * (c / (8 * C::CODE_BLK));
      }
      constexpr int kQStepPad = C::QSTEP + 8 * (C::QSTEP / (8 * C::CODE_BLK));
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        const int cu = cpad[q & 3] + kQStepPad * (q >> 2);
        float t[BW];
#pragma unroll
        for (int k = 0; k < BW; ++k) t[k] = magic_code<CLAMP>(v[BW * q + k], kq);
        // byte 0 of each magic word is q + 8 (four bits); xor 8 gives the
        // two's complement nibble
        const uint32_t ev = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, t[2]),
                                                  __builtin_bit_cast(uint32_t, t[0]), 0x0c0c0400u);
        const uint32_t od = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, t[3]),
                                                  __builtin_bit_cast(uint32_t, t[1]), 0x0c0c0400u);
        reinterpret_cast<uint16_t*>(buf + C::CODE_OFF)[cu] =
            uint16_t((((od << 4) | ev) ^ 0x8888u) & 0xFFFFu);
      }
      if (x_rot) {
        float* xr = x_rot + row * int64_t(C::D) + abase * M + BW * unit;
#pragma unroll
        for (int q = 0; q < QN; ++q)
#pragma unroll
          for (int k = 0; k < BW; ++k)
            xr[M * (4 * (q & 3) + 128 * (q >> 2)) + k] = v[BW * q + k] * norm;
      }
    }
    return s16;
  };
  // the row's codes: D / 2 bytes from the LDS code area, 16-byte stores
  auto store_codes = [&](int64_t row, __half s16) {
    uint8_t* qrow = q_out + row * ld_q;
    constexpr int kChunks = C::D / 32, kIter = (kChunks + C::THREADS - 1) / C::THREADS;
#pragma unroll
    for (int i = 0; i < kIter; ++i) {
      const int c = tid + C::THREADS * i;
      if (i + 1 < kIter || c < kChunks)
        *reinterpret_cast<uint4*>(qrow + 16 * c) =
            reinterpret_cast<const uint4*>(buf + C::CODE_OFF)[c + c / C::CODE_BLK];
    }
    if (tid == 0) scale_out[row] = s16;
  };

  int64_t row = blockIdx.x;
  uint4 raw[NR], raw_u[TU];
  if (row >= rows) return;
  load_row(row, raw, raw_u);
  // One row at a time, two barriers per row.  A row's codes leave after the
  // next row's first barrier (or after the loop): every thread has written
  // them by then, and every thread has read them before it reaches the next
  // row's second barrier, after which that row's codes take the area.  red
  // is read between a row's second barrier and the next row's first, and
  // written between those two.
  int64_t prev = -1;  // the row whose codes wait in the LDS code area
  __half prev_s16 = __half(0.0f);
  for (; row < rows; row += gridDim.x) {
    float v[8 * TILES];
    const int64_t nrow = row + gridDim.x;
    phase1(raw, raw_u, v, nrow);
    if (!SWIGLU && nrow < rows) load_row(nrow, raw, raw_u);  // prefetch
    write_row(v);
    __syncthreads();
    if (prev >= 0) store_codes(prev, prev_s16);
    // phase 2 reuses the registers
    float(&v2)[NV] = *reinterpret_cast<float(*)[NV]>(&v[0]);
    float amax = phase2(v2);
    amax = wave_max_dpp(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();  // phase-2 reads of buf are done; red is complete
    prev_s16 = quantize(v2, row);
    prev = row;
  }
  __syncthreads();
  store_codes(prev, prev_s16);
}

}  // namespace quarot
