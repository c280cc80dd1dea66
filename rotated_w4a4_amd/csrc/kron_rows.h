// Rotate+quant of rows of d = NP * m (H_NP (x) H_m, NP = 2^n): one
// workgroup owns one row (NP = 1024: 512 threads, one per CU; NP = 512: 256
// threads, two per CU, so two rows are in flight per CU).  H_m is the
// caller's matrix, handed in as bit masks.  d = 28672 (plain and gated) runs
// here as 1024 groups of 28.  The rows of 512 groups (d = 12288 as groups of
// 24 under H_2 (x) H_12) are dispatched to had_quant_kront, which keeps every
// butterfly in registers; the NP = 512 configuration below is the layout
// that kernel replaced.
//
// With SWIGLU the row is the gated FFN product c = SiLU(gate) * up, formed
// in fp32 from the two fp16 inputs as they arrive (the same page, section
// 3.4 Stage 1b: the online Hadamard acts on that product).  The matrix cores
// take fp16 operands, so c is split into hi = fp16(c) and
// lo = fp16((c - hi) * 2^11); H_m hi and (2^-11 H_m) lo accumulate in fp32
// (products exact), keeping about 22 bits of c.
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary), section 3.4 Stage 1a: for d = 2^n m the Hadamard is
// H_{2^n} (x) H_m with a known H_m, computable in O(d (m + n)); Stage 1b:
// the online Hadamard before the down-projection (d = 28672 is the
// LLaMA2-70B down-projection input, d = 12288 the Qwen3-8B one, which the
// QuaRot paper-viz explainer builds with a Paley-12 block).
//
// Element e = a * m + b, a = 0..NP-1 (the power-of-two index), b = 0..m-1.
//   phase 1  wave w (of W = 8 or 4), lane l = n + 16 g, tile t (of NP /
//            (16 W)) hold group a = (NP / W) w + 16 t + n.  The lane loads
//            elements b = 8 g .. 8 g + 7 of its group (zero past m) with one
//            16-byte load inside the group: the B operand of
//            v_mfma_f32_16x16x32_f16.  H_m (rows 0-15 and, for m > 16,
//            16-31; zero padded to 32 x 32) is the A operand, so the dense
//            H_m factor runs on the matrix cores on the raw sign-flipped fp16
//            input (products with +-1 are exact, sums fp32).  The output
//            lands as b = 4 g + (0..3) and 16 + 4 g + (0..3).  Butterflies
//            over a4-a6 (tile t) run in registers, over a0, a1, a3 (lane bits
//            0, 1, 3) through DPP.  Valid outputs go to LDS as fp32.
//   phase 2  task (c, u): c fixes a0, a1, a3, a4, a5, a6, u a run of BW
//            consecutive b.  The task reads its BW values of each of the
//            QN = NP / 64 groups that differ in a2 and a7 up (float4 reads),
//            runs those butterfly stages in registers, joins the workgroup
//            maximum, quantises and writes 16- or 32-bit code units to LDS;
//            the row's codes then leave in 16-byte stores.
#pragma once

#include "wave_rows.h"

namespace quarot {

// Entry c of a mask row (already shifted to the lane's first column).
__device__ __forceinline__ _Float16 had_entry(uint32_t nz, uint32_t neg, int c) {
  if (!((nz >> c) & 1u)) return _Float16(0.0f);
  return ((neg >> c) & 1u) ? _Float16(-1.0f) : _Float16(1.0f);
}

// Row r of the masks for a lane-dependent r < 32: the kernel argument is
// read with uniform loads and selected per lane.
__device__ __forceinline__ uint32_t mask_row(const uint32_t (&rowsv)[32], int r) {
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) out = (r == i) ? rowsv[i] : out;
  return out;
}

// SiLU(t) = t / (1 + exp(-t)) in fp32: v_exp_f32 (2^x) and v_rcp_f32, each
// within about one ulp.  For t -> -inf the exponential overflows to inf and
// the result is -0; for t -> +inf it is t.
__device__ __forceinline__ float silu_f32(float t) {
  const float e = __builtin_amdgcn_exp2f(t * -1.4426950408889634f);
  return t * __builtin_amdgcn_rcpf(1.0f + e);
}

// Eight gated products c = SiLU(g) u from one 16-byte chunk of each input,
// split for the matrix cores: hi = fp16(c), lo = fp16((c - hi) * 2^11).
// The element's random sign is already in u (its fp16 sign bit flipped).
// c = (g u) / (1 + 2^(-g log2 e)): g u is exact in fp32 (two fp16 factors),
// so c takes one rounding.  c is made opaque once formed, and the residual
// c - hi (exact) is taken from the very fp16 pair that feeds the MFMA: the
// backend would otherwise fold fp16(c) into a single-rounding multiply for
// the residual while the operand takes fp16 of the rounded product, and
// where the two disagree by an fp16 ulp the low part no longer completes hi.
__device__ __forceinline__ void swiglu_split8(const uint4& g, const uint4& u, uint4& hi,
                                              uint4& lo) {
  typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
  const half8_t gh = __builtin_bit_cast(half8_t, g);
  const half8_t uh = __builtin_bit_cast(half8_t, u);
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float c[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = 2 * k + i;
      // (each product written as an fma of widened fp16 operands, so it runs
      // as one mixed-precision fma with no separate conversions)
      const float e = __builtin_amdgcn_exp2f(
          __builtin_fmaf(static_cast<float>(gh[j]), -1.4426950408889634f, 0.0f));
      const float p = __builtin_fmaf(static_cast<float>(gh[j]), static_cast<float>(uh[j]), 0.0f);
      c[i] = p * __builtin_amdgcn_rcpf(1.0f + e);
      asm volatile("" : "+v"(c[i]));
    }
    const half2_t hp = {static_cast<_Float16>(c[0]), static_cast<_Float16>(c[1])};
    hw[k] = __builtin_bit_cast(uint32_t, hp);
    // c - hi, exact, from the packed hi pair itself (one mixed fma per value)
    float r0, r1;
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r0) : "v"(hw[k]), "v"(c[0]));
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=v"(r1) : "v"(hw[k]), "v"(c[1]));
    const half2_t lp = {static_cast<_Float16>(r0 * 2048.0f), static_cast<_Float16>(r1 * 2048.0f)};
    lw[k] = __builtin_bit_cast(uint32_t, lp);
  }
  hi = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  lo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
}

// LDS row of group a: a2 is flipped when a4 is set.  Phase 1 writes 16
// consecutive groups per LDS cycle, phase 2 reads groups that differ in a0,
// a1, a3, a4; with rows of m floats (m / 4 odd) both hit 16 distinct float4
// bank slots.
__device__ __forceinline__ int kron_row(int a) { return a ^ (((a >> 4) & 1) << 2); }

// One butterfly stage over lane bit 0, 1 or 3 (STAGE 0, 1, 2) on the phase-1
// registers, as v + partner * c in a single v_fmac_f32 with DPP (c = +1 on the
// low lane, -1 on the high lane, so a high lane ends with b - a).  HALVES == 1
// skips the registers of the unused upper MFMA half.
//
// DPP reads need two wait states after a VALU write of their source.  Stage 0
// reads registers written by compiler-scheduled code, so each of its blocks
// opens with s_nop 1; stages 1 and 2 read only what the previous stage's asm
// blocks wrote, at least 28 instructions earlier.  The last block of stage 2
// closes with s_nop 1 for whatever follows.
template <int STAGE, int HALVES, int N>
__device__ __forceinline__ void dpp_fmac_stage(float (&v)[N], float c) {
#define QR_FMAC_DPP(LEAD, CTRL, TRAIL)                                                       \
  asm volatile(LEAD                                                                          \
               "v_fmac_f32_dpp %0, %0, %4 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               "v_fmac_f32_dpp %1, %1, %4 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               "v_fmac_f32_dpp %2, %2, %4 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               "v_fmac_f32_dpp %3, %3, %4 " CTRL " row_mask:0xf bank_mask:0xf" TRAIL      \
               : "+v"(v[r]), "+v"(v[r + 1]), "+v"(v[r + 2]), "+v"(v[r + 3])              \
               : "v"(c))
  constexpr int kLast = HALVES == 1 ? N - 8 : N - 4;
#pragma unroll
  for (int r = 0; r < N; r += 4) {
    if (HALVES == 1 && (r & 4)) continue;
    if (STAGE == 0) QR_FMAC_DPP("s_nop 1\n", "quad_perm:[1,0,3,2]", "");
    else if (STAGE == 1) QR_FMAC_DPP("", "quad_perm:[2,3,0,1]", "");
    else if (r != kLast) QR_FMAC_DPP("", "row_ror:8", "");
    else QR_FMAC_DPP("", "row_ror:8", "\ns_nop 1");
  }
#undef QR_FMAC_DPP
}

// A row of d = NP m elements: NP = 2^n groups of m.  The plain d = 12288 row
// is taken as 512 groups of 24 under H_24 = H_2 (x) H_12 (the Sylvester
// H_1024 is H_512 (x) H_2, so H_1024 (x) H_12 = H_512 (x) H_24): the
// matrix cores then apply 24 of their 32 K slots instead of 12.
template <int M, bool SWIGLU = false, int NP = 1024>
struct KronCfg {
  static constexpr int D = NP * M;
  // A wave owns 128 groups in phase 1 (eight tiles of 16 per lane).  NP =
  // 512 (d = 12288): 256-thread blocks (four waves), two blocks per CU, so
  // two rows are in flight per CU with their own barriers and prefetches;
  // NP = 1024 (d = 28672: 112 KiB of fp32 in LDS) takes the whole CU: one
  // 512-thread block of eight waves.
  static constexpr int AW = 128;  // groups per wave in phase 1
  static constexpr int TILES = AW / 16;
  static constexpr int NWAVE = NP / AW;
  static constexpr bool TWO_BLOCKS = NWAVE == 4;
  static constexpr int THREADS = 64 * NWAVE;
  static constexpr int BLOCKS_PER_CU = TWO_BLOCKS ? 2 : 1;
  // phase 2: a task owns QN groups (the group bits left after phase 1) and
  // a run of BW consecutive b of each: 64 values
  static constexpr int QN = NP / 64;
  static constexpr int BW = 64 / QN;
  static constexpr int UNITS = M / BW;      // runs of BW consecutive b per group
  static constexpr int TASKS = 64 * UNITS;  // phase-2 tasks per row
  static constexpr int HALVES = (M > 16) ? 2 : 1;
  // LDS row stride in floats: an odd number of float4 slots, so that both
  // exchange patterns hit 16 distinct bank slots (m = 24 is padded to 28)
  static constexpr int RS = ((M / 4) % 2 == 1) ? M : M + 4;
  static constexpr int CODE_OFF = NP * RS;  // the codes follow the fp32 row
  static constexpr int LDS_BYTES = CODE_OFF * 4 + D / 2;
  // Register-lean addressing for the gated product (two input streams):
  // buffer loads over the row (one 32-bit lane offset instead of a 64-bit
  // address per tile and stream) and phase-2 addresses recomputed per row
  // from an opaque base.  The plain rows keep global loads and let the
  // compiler hoist the addresses, which measured faster for m = 28.
  static constexpr bool LEAN = SWIGLU;
  // The gated product is formed on a compact layout: a wave's groups (AW of
  // them, contiguous in the row) are J 16-byte chunks per lane and stream,
  // every element real, where the MFMA operand layout pads each group of m
  // to 32 slots (m = 24: 24 of 32, m = 28: 28 of 32).  The products' hi and
  // lo parts go through the wave's own rows of the LDS row area and are
  // read back in the operand layout.
  static constexpr int J = SWIGLU ? AW * M / 512 : 1;
  static_assert(!SWIGLU || AW * M % 512 == 0, "whole chunks per lane");
  static_assert(M % 4 == 0 && M <= 32 && M % BW == 0, "m must be a multiple of 4 up to 32");
  static_assert(NP == 512 || NP == 1024, "four or eight waves per row");
  static_assert(TASKS <= THREADS, "one phase-2 task per thread");
};

// SWIGLU: x is the gate projection and up the up projection; the row is
// SiLU(x) * up.  Otherwise up is unused and the row is x.
template <int M, bool CLAMP, bool SWIGLU, int NP>
__global__ __launch_bounds__((KronCfg<M, SWIGLU, NP>::THREADS), 2) void had_quant_kron(
    const __half* __restrict__ x, int64_t ld_x, const __half* __restrict__ up, int64_t ld_up,
    int64_t rows, const int8_t* __restrict__ signs, HadMasks hm, float clip_ratio,
    uint8_t* __restrict__ q_out, int64_t ld_q, __half* __restrict__ scale_out,
    float* __restrict__ x_rot, float norm) {
  using C = KronCfg<M, SWIGLU, NP>;
  extern __shared__ float4 kron_lds[];  // the row in fp32 (phase 1 -> phase 2), then its codes
  float* buf = reinterpret_cast<float*>(kron_lds);
  __shared__ float red[C::NWAVE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;

  // valid elements of this lane's chunk of a group: b = 8 g .. 8 g + cnt - 1
  // (cnt is 8 or 0 for m = 24; 8 or 4 for m = 28)
  const int cnt = min(8, max(0, M - 8 * g));
  // Each lane loads 16 bytes (8 elements) of its group in one instruction,
  // always inside the group: a full chunk (cnt = 8) at b = 8 g; a half chunk
  // (cnt = 4, the group's last four elements) at b = 8 g - 4, so the wanted
  // values sit in the upper half; lanes past m at the group start.  The
  // slots that are not wanted meet zero columns of the A operand: they hold
  // other elements of the same group, so with finite inputs they add exact
  // zeros (a non-finite input spoils its group's outputs either way).
  const int off16 = cnt == 8 ? 8 * g : (cnt == 4 ? 8 * g - 4 : 0);
  // A operands: H_m rows n (and 16 + n) against the lane's K slots, zero
  // padded: slot j pairs with column 8 g + j, or 8 g + j - 4 for a half chunk.
  const int shift = (cnt == 4 && !SWIGLU) ? 4 : 0;
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
  // signs of this lane's phase-1 elements (the same for every row), as fp16
  // sign-bit masks: group a = 128 wave + 16 t + n
  constexpr int TILES = C::TILES, AW = C::AW, J = C::J, RS = C::RS;
  uint4 mask[SWIGLU ? 1 : TILES];
  // gated product: the fp16 sign-bit masks of compact chunk j, XORed into up
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
  const float s_q1 = (lane & 1) ? -1.0f : 1.0f;
  const float s_q2 = (lane & 2) ? -1.0f : 1.0f;
  const float s_r8 = (lane & 8) ? -1.0f : 1.0f;

  // phase-2 task of this thread
  const bool task_on = tid < C::TASKS;
  const int combo = tid & 63, unit = tid >> 6;
  const int abase = (combo & 3) + (((combo >> 2) & 1) << 3) + (((combo >> 3) & 7) << 4);
  // sign left on this task's values by the phase-1 DPP stages
  const float sigma = (__builtin_popcount(combo & 7) & 1) ? -1.0f : 1.0f;

  // loads of one row's phase-1 chunks (the up projection's too when gated;
  // LEAN: buffer loads, tile t at lane offset + 32 m bytes).  (The lanes past
  // m are masked at use: masking here would make the prefetch wait for its
  // own data.)
  constexpr int NR = SWIGLU ? J : TILES, TU = SWIGLU ? J : 1;
  const int lane_off =
      SWIGLU ? 2 * (AW * wave * M + 8 * lane) : 2 * ((AW * wave + n) * M + off16);
  // byte step between a lane's loads: compact chunks, or tiles of 16 groups
  constexpr int LSTEP = SWIGLU ? 1024 : 32 * M;
  // one compact chunk of both inputs of the gated product
  auto load_chunk = [&](int64_t row, int j, uint4& r, uint4& ru) {
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<__half*>(x + row * ld_x), 0, 2 * C::D,
                                          0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<__half*>(up + row * ld_up), 0, 2 * C::D,
                                          0x00020000);
    r = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, lane_off + LSTEP * j, 0, 0));
    ru = __builtin_bit_cast(uint4,
                            __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off + LSTEP * j, 0, 0));
  };
  auto load_row = [&](int64_t row, uint4 (&raw)[NR], uint4 (&raw_u)[TU]) {
    if constexpr (!C::LEAN) {
      const __half* src = x + row * ld_x;
#pragma unroll
      for (int t = 0; t < TILES; ++t)
        __builtin_memcpy(&raw[t], src + (AW * wave + 16 * t + n) * M + off16, 16);
      return;
    }
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<__half*>(x + row * ld_x), 0, 2 * C::D,
                                          0x00020000);
#pragma unroll
    for (int t = 0; t < NR; ++t)
      raw[t] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, lane_off + LSTEP * t, 0, 0));
    if constexpr (SWIGLU) {
      const __amdgpu_buffer_rsrc_t ru =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<__half*>(up + row * ld_up), 0, 2 * C::D,
                                            0x00020000);
#pragma unroll
      for (int t = 0; t < J; ++t)
        raw_u[t] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(ru, lane_off + LSTEP * t, 0, 0));
    }
  };

  // ---- phase 1: H_m on the matrix cores, then the butterflies over a4-a6
  // (register bits) and a0, a1, a3 (lane bits, DPP) -------------------------
  // (gated product: nrow < rows issues the next row's loads chunk by chunk
  // as soon as each chunk's registers are free, so they overlap the long
  // product phase instead of following it)
  auto phase1 = [&](uint4 (&raw)[NR], uint4 (&raw_u)[TU], float (&v)[8 * TILES],
                    int64_t nrow) {
    if constexpr (SWIGLU) {
      // products, signs and the hi / lo split on the compact chunks, staged
      // in this wave's rows of the LDS row area: hi parts, then lo parts
      _Float16* shi = reinterpret_cast<_Float16*>(buf + AW * wave * RS);
      _Float16* slo = shi + AW * M;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint4 um = make_uint4(raw_u[j].x ^ cmask[j].x, raw_u[j].y ^ cmask[j].y,
                                    raw_u[j].z ^ cmask[j].z, raw_u[j].w ^ cmask[j].w);
        uint4 hi, lo;
        swiglu_split8(raw[j], um, hi, lo);
        if (nrow < rows) load_chunk(nrow, j, raw[j], raw_u[j]);
        *reinterpret_cast<uint4*>(shi + 512 * j + 8 * lane) = hi;
        *reinterpret_cast<uint4*>(slo + 512 * j + 8 * lane) = lo;
      }
      // the wave reads back what its own lanes wrote: LDS completes a wave's
      // accesses in order once they have all been issued and counted
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
      float4_t d0, d1 = zero;
      if constexpr (SWIGLU) {
        // operand slots j < cnt hold b = 8 g + j of group 16 t + n
        const _Float16* shi = reinterpret_cast<const _Float16*>(buf + AW * wave * RS);
        const _Float16* slo = shi + AW * M;
        const int e = (16 * t + n) * M + (cnt > 0 ? 8 * g : 0);
        uint4 hi, lo;
        if constexpr (M % 8 == 0) {
          // whole chunks (16-byte aligned); lanes past m read their group's
          // first chunk, against zero columns of H
          hi = *reinterpret_cast<const uint4*>(shi + e);
          lo = *reinterpret_cast<const uint4*>(slo + e);
        } else {
          // two 8-byte halves; slots past cnt are zeroed (a half chunk's
          // upper slots would reach the next group, or past the wave's
          // staging rows)
          const uint2 h0 = *reinterpret_cast<const uint2*>(shi + e);
          const uint2 h1 = *reinterpret_cast<const uint2*>(shi + e + 4);
          const uint2 q0 = *reinterpret_cast<const uint2*>(slo + e);
          const uint2 q1 = *reinterpret_cast<const uint2*>(slo + e + 4);
          const uint32_t k_lo = cnt > 0 ? 0xFFFFFFFFu : 0u;   // slots 0-3
          const uint32_t k_hi = cnt == 8 ? 0xFFFFFFFFu : 0u;  // slots 4-7
          hi = make_uint4(h0.x & k_lo, h0.y & k_lo, h1.x & k_hi, h1.y & k_hi);
          lo = make_uint4(q0.x & k_lo, q0.y & k_lo, q1.x & k_hi, q1.y & k_hi);
        }
        const half8_t bh = __builtin_bit_cast(half8_t, hi);
        const half8_t bl = __builtin_bit_cast(half8_t, lo);
        // H_m hi, then 2^-11 H_m lo accumulated onto it (exact products)
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(h_lo, bh, zero, 0, 0, 0);
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(hs_lo, bl, d0, 0, 0, 0);
        if (C::HALVES == 2) {
          d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(h_hi, bh, zero, 0, 0, 0);
          d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(hs_hi, bl, d1, 0, 0, 0);
        }
        // one tile's products at a time: interleaving the tiles' conversions
        // would hold several tiles' temporaries at once and spill
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // (the gated product's signs are applied on its compact chunks)
        const uint4 r = make_uint4(raw[t].x ^ mask[t].x, raw[t].y ^ mask[t].y,
                                   raw[t].z ^ mask[t].z, raw[t].w ^ mask[t].w);
        const half8_t bop = __builtin_bit_cast(half8_t, r);
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(h_lo, bop, zero, 0, 0, 0);
        if (C::HALVES == 2) d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(h_hi, bop, zero, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[8 * t + q] = d0[q];
        v[8 * t + 4 + q] = d1[q];
      }
    }
  };
  auto butterflies1 = [&](float (&v)[8 * TILES]) {
    // a4-a6: register bits 3-5
#pragma unroll
    for (int h = 8; h < 64; h <<= 1)
#pragma unroll
      for (int r = 0; r < 8 * TILES; ++r)
        if ((r & h) == 0) {
          const float a = v[r], b = v[r + h];
          v[r] = a + b;
          v[r + h] = a - b;
        }
    // a0, a1, a3: lane bits 0, 1, 3 through DPP
    // (one v_fmac_f32_dpp each: a high lane keeps b - a, so after the three
    // stages lane values carry the sign (-1)^(a0 + a1 + a3), undone in phase 2)
    dpp_fmac_stage<0, C::HALVES>(v, s_q1);
    dpp_fmac_stage<1, C::HALVES>(v, s_q2);
    dpp_fmac_stage<2, C::HALVES>(v, s_r8);
  };
  // valid phase-1 outputs to LDS: b = 16 h + 4 g + (0..3), group a at row
  // kron_row(a)
  auto write_row = [&](const float (&v)[8 * TILES]) {
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int a = kron_row(AW * wave + 16 * t + n);
#pragma unroll
      for (int h = 0; h < C::HALVES; ++h) {
        const int b0 = 16 * h + 4 * g;
        if (b0 < M)
          *reinterpret_cast<float4*>(buf + a * RS + b0) =
              make_float4(v[8 * t + 4 * h], v[8 * t + 4 * h + 1], v[8 * t + 4 * h + 2],
                          v[8 * t + 4 * h + 3]);
      }
    }
  };
  // ---- phase 2: a2 and the group bits from a7 up, in registers ----------
  // register r = BW q + i holds b = BW unit + i of group a(q), q < QN.
  // Group a(q) = abase + 4 (q & 1) + 128 (q >> 1); its LDS row
  // kron_row(a(q)) flips bit 2 when bit 4 of abase is set.  With LEAN the
  // per-thread base is made opaque per row, so the addresses are base +
  // constant in the loop rather than registers kept across it.  Returns the
  // task's largest |value| (0 for threads without a task).
  constexpr int BW = C::BW, QN = C::QN, NV = QN * BW;
  auto phase2 = [&](float (&v)[NV]) -> float {
    float amax = 0.0f;
    int tbase = abase * RS + BW * unit;
    if (C::LEAN) asm volatile("" : "+v"(tbase));
    const int flip4 = ((abase >> 4) & 1) ? 4 * RS : 0;
    if (task_on) {
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        const int a_off = ((q & 1) ? 4 * RS - flip4 : flip4) + 128 * RS * (q >> 1);
#pragma unroll
        for (int k = 0; k < BW; k += 4) {
          const float4 f = *reinterpret_cast<const float4*>(buf + tbase + a_off + k);
          v[BW * q + k] = f.x;
          v[BW * q + k + 1] = f.y;
          v[BW * q + k + 2] = f.z;
          v[BW * q + k + 3] = f.w;
        }
      }
#pragma unroll
      for (int h = BW; h < NV; h <<= 1)
#pragma unroll
        for (int r = 0; r < NV; ++r)
          if ((r & h) == 0) {
            const float a = v[r], b = v[r + h];
            v[r] = a + b;
            v[r + h] = a - b;
          }
#pragma unroll
      for (int r = 0; r < NV; ++r) amax = fmaxf(amax, fabsf(v[r]));
    }
    return amax;
  };
  // the row's scale from the per-wave maxima in red, then its codes to the
  // LDS code area (BW codes per unit: 16 or 32 bits), and the optional fp32
  // copy.  The element offset of register q's run in the row (natural
  // order) is ebase + M (4 (q & 1) + 128 (q >> 1)), a multiple of BW.
  auto quantize = [&](const float (&v)[NV], int64_t row) -> __half {
    float amax = red[0];
#pragma unroll
    for (int w = 1; w < C::NWAVE; ++w) amax = fmaxf(amax, red[w]);
    const __half s16 = row_scale_fp16(amax * norm, clip_ratio);
    const float kq = inv_scale(s16) * norm * sigma;
    if (task_on) {
      int cbase = abase * (M / BW) + unit;  // code unit of register 0's run
      if (C::LEAN) asm volatile("" : "+v"(cbase));
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        const int cu = cbase + (M / BW) * (4 * (q & 1) + 128 * (q >> 1));
        float t[BW];
#pragma unroll
        for (int i = 0; i < BW; ++i) t[i] = magic_code<CLAMP>(v[BW * q + i], kq);
        if constexpr (BW == 8) {
          reinterpret_cast<uint32_t*>(buf + C::CODE_OFF)[cu] = pack8_magic(t);
        } else {
          const uint32_t ev = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, t[2]),
                                                    __builtin_bit_cast(uint32_t, t[0]), 0x0c0c0400u);
          const uint32_t od = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, t[3]),
                                                    __builtin_bit_cast(uint32_t, t[1]), 0x0c0c0400u);
          reinterpret_cast<uint16_t*>(buf + C::CODE_OFF)[cu] =
              uint16_t((((od << 4) | ev) ^ 0x8888u) & 0xFFFFu);
        }
      }
      if (x_rot) {
        const float xnorm = norm * sigma;
        float* xr = x_rot + row * int64_t(C::D) + BW * cbase;
#pragma unroll
        for (int q = 0; q < QN; ++q)
#pragma unroll
          for (int k = 0; k < BW; k += 4)
            *reinterpret_cast<float4*>(xr + M * (4 * (q & 1) + 128 * (q >> 1)) + k) =
                make_float4(v[BW * q + k] * xnorm, v[BW * q + k + 1] * xnorm,
                            v[BW * q + k + 2] * xnorm, v[BW * q + k + 3] * xnorm);
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
            reinterpret_cast<const uint4*>(buf + C::CODE_OFF)[c];
    }
    if (tid == 0) scale_out[row] = s16;
  };

  int64_t row = blockIdx.x;
  uint4 raw[NR], raw_u[TU];
  if (row >= rows) return;
  load_row(row, raw, raw_u);
  // One row at a time: phase 1, the next row's loads, LDS, phase 2, codes.
  // Two barriers per row.  A row's codes leave after the next row's first
  // barrier (or after the loop): every thread has written them by then, and
  // every thread has read them before it reaches the next row's second
  // barrier, after which that row's codes overwrite the area.  red is safe
  // the same way: it is read between a row's second barrier and the next
  // row's first, written between those two.
  // (Running phase 1 of the next row inside phase 2 of this one, two rows in
  // flight per workgroup, measured slower: the kernel is bound by VALU issue,
  // not by the latency between phases.)
  int64_t prev = -1;  // the row whose codes wait in the LDS code area
  __half prev_s16 = __half(0.0f);
  for (; row < rows; row += gridDim.x) {
    float v[8 * TILES];
    const int64_t nrow = row + gridDim.x;
    phase1(raw, raw_u, v, nrow);
    if (!SWIGLU && nrow < rows) load_row(nrow, raw, raw_u);  // prefetch
    butterflies1(v);
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
