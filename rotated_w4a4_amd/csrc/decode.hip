// quarot_kv_decode_attention: one decode step of attention over the INT4
// KV cache written by quarot_kv_had_quant.
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary), section 3.4: Stage 1d (the new query is rotated head-wise by the
// same Hadamard as the cached keys, so the scores q k^T are unchanged;
// softmax(q k^T / sqrt(d_h))), Stage 2c (at decode every cached group is
// dequantised on the fly) and Stage 1c (the online cross-head transform
// Z (H_{n_h} (x) I_{d_h}) on the attention output before the output
// projection).
//
// Two kernels:
//   decode_split_kernel    one workgroup per (batch, KV head, position split)
//                          with all query heads of the KV head's group
//                          (<= 8): rotate the queries (signs, FWHT-128 by
//                          shuffles), then per wave a loop over 32-position
//                          steps with an online softmax; scores and P V run
//                          on v_mfma_f32_16x16x32_f16 with the fp32 operand
//                          split into fp16 hi + lo rows (products of fp16
//                          values with small integers are exact, so the result
//                          keeps about 22 bits).  Writes (max, sum, unscaled
//                          output) per split.
//   decode_combine_kernel  merges the splits, divides by the softmax sum,
//                          optionally applies the cross-head Walsh-Hadamard
//                          transform over the query heads, writes fp16.
//
// Operand layouts of v_mfma_f32_16x16x32_f16 (lane = column + 16 * group):
//   A[m][k] at lane m + 16 (k / 8), item k % 8; B[k][n] at lane n + 16 (k / 8),
//   item k % 8; D[m][n] at lane n + 16 (m / 4), item m % 4.
// A rows are (head, part) pairs: row m = head m / 2, part m % 2 (0 hi, 1 lo),
// so a D lane holds hi and lo of two heads side by side.
//
// Nibbles become fp16 as (1024 + u) - offset: OR-ing a nibble u into the
// mantissa of 1024.0 and subtracting 1024 + 8 (two's complement codes,
// flipped to offset binary first) or 1024 + z (zero-point codes); both steps
// are exact.  The 8 nibbles of a dword come out in the order
// 0, 4, 1, 5, 2, 6, 3, 7, and the other operand uses the same order.
#include <atomic>
#include <mutex>

#include "decode.h"
#include "wave_rows.h"

namespace quarot {

namespace {

constexpr int kDecD = 128;
constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecStep = 32;    // positions per wave step
constexpr int kDecHeads = 8;    // query heads per KV head (at most)
constexpr int kDecUnit = kDecWaves * kDecStep;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

struct DecodeArgs {
  const __half* q;  // [B, Hq, 128]
  const int8_t* signs;
  int64_t signs_stride_h;
  const uint8_t* kq;
  const __half* ks;
  const __half* kz;
  const uint8_t* vq;
  const __half* vs;
  const __half* vz;
  int hkv, hq, group;
  int64_t s_cache;
  int max_len;
  const int32_t* lengths;
  int splits, split_len;
  float score_mul;  // softmax scale * log2(e)
  float* part_o;    // [B * Hkv * splits][group][128]
  float* part_ml;   // [B * Hkv * splits][group][2]: running max (log2 units), sum
};

// k-slot s of an 8-value operand holds nibble / element perm8(s).
__device__ __forceinline__ constexpr int perm8(int s) { return (s >> 1) + 4 * (s & 1); }

// Slots 2, 3, 6, 7 (nibbles 1, 5, 3, 7) are taken from bits 4..7 of a
// halfword, i.e. at 16 times their value; the other operand divides those
// slots by 16 (a power of two: exact).
__device__ __forceinline__ constexpr bool slot_x16(int s) { return (s & 2) != 0; }

// (x & m) ^ c on the bits of m, c elsewhere: v_bitop3 with table 0x6A.  With
// c = the fp16 exponent of 1024 outside m and an XOR pattern inside m it
// builds 1024 + u (or 1024 + 16 u) straight from a nibble, flipping
// two's-complement codes to offset binary on the way when asked.
__device__ __forceinline__ uint32_t nib_bits(uint32_t x, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(x, m, c, 0x6A);
}

// 8 nibbles -> 8 exact fp16 values in slot order perm8:
//   slots 0, 1, 4, 5: (1024 + u) - off1 ;  slots 2, 3, 6, 7: (1024 + 16 u) - off16,
// with u the nibble, XOR 8 when FLIP (two's complement -> offset binary).
template <bool FLIP>
__device__ __forceinline__ half8_t nibbles_to_half8(uint32_t w, half2_t off1, half2_t off16) {
  constexpr uint32_t kLo = 0x000F000Fu, kHi = 0x00F000F0u;
  constexpr uint32_t cLo = 0x64006400u | (FLIP ? 0x00080008u : 0u);
  constexpr uint32_t cHi = 0x64006400u | (FLIP ? 0x00800080u : 0u);
  const uint32_t w8 = w >> 8;
  const half2_t h0 = __builtin_bit_cast(half2_t, nib_bits(w, kLo, cLo)) - off1;     // nibbles 0, 4
  const half2_t h1 = __builtin_bit_cast(half2_t, nib_bits(w, kHi, cHi)) - off16;    // 1, 5
  const half2_t h2 = __builtin_bit_cast(half2_t, nib_bits(w8, kLo, cLo)) - off1;    // 2, 6
  const half2_t h3 = __builtin_bit_cast(half2_t, nib_bits(w8, kHi, cHi)) - off16;   // 3, 7
  half8_t r;
  r[0] = h0[0];
  r[1] = h0[1];
  r[2] = h1[0];
  r[3] = h1[1];
  r[4] = h2[0];
  r[5] = h2[1];
  r[6] = h3[0];
  r[7] = h3[1];
  return r;
}

// 8 x 8 nibble transpose: on entry nibble j of r[i] is element (i, j), on
// exit nibble i of r[j].  Three exchanges of index bits: bit 2 (halfwords),
// bit 1 (bytes), bit 0 (nibbles), each between a pair of registers.
__device__ __forceinline__ void transpose_nibbles8(uint32_t (&r)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = r[i], b = r[i + 4];
    r[i] = __builtin_amdgcn_perm(b, a, 0x05040100u);      // a.lo16 | b.lo16 << 16
    r[i + 4] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // a.hi16 | b.hi16 << 16
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if ((i & 2) == 0) {
      const uint32_t a = r[i], b = r[i + 2];
      r[i] = __builtin_amdgcn_perm(b, a, 0x06020400u);      // bytes a0 b0 a2 b2
      r[i + 2] = __builtin_amdgcn_perm(b, a, 0x07030501u);  // bytes a1 b1 a3 b3
    }
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const uint32_t a = r[i], b = r[i + 1];
    r[i] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
    r[i + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  }
}

// Maximum over each row of 16 lanes, for two values at once: each stage is
// one v_max_f32 with a DPP row rotation on its first operand.  The two chains
// alternate, and an s_nop 0 between pairs completes the two wait states a
// DPP read needs after the VALU write of its source.
__device__ __forceinline__ void row_max16x2(float& a, float& b) {
  asm volatile(
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "v_max_f32_dpp %1, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      "s_nop 0\n"
      "v_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "v_max_f32_dpp %1, %1, %1 row_ror:4 row_mask:0xf bank_mask:0xf\n"
      "s_nop 0\n"
      "v_max_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf\n"
      "v_max_f32_dpp %1, %1, %1 row_ror:2 row_mask:0xf bank_mask:0xf\n"
      "s_nop 0\n"
      "v_max_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf\n"
      "v_max_f32_dpp %1, %1, %1 row_ror:1 row_mask:0xf bank_mask:0xf\n"
      "s_nop 1"
      : "+v"(a), "+v"(b));
}

__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_mov<0x128>(v);
  v += dpp_mov<0x124>(v);
  v += dpp_mov<0x122>(v);
  v += dpp_mov<0x121>(v);
  return v;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer over [base, base + bytes): loads at offsets >= bytes return 0
// and touch no memory.
__device__ __forceinline__ rsrc_t buffer_of(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Per workgroup: buffers over the split's positions [0, pos_end) of its
// (batch, KV head) cache rows.
struct SplitBuffers {
  rsrc_t k, v, ks, vs, kz, vz;
};

// One step's loads for a lane.  K: lane (n, g) holds bytes 16 g .. 16 g + 15
// (head dims 32 g .. 32 g + 31) of positions base + n and base + 16 + n.
// V: lane (c, g) holds dword c (dims 8 c .. 8 c + 7) of positions
// base + g + 4 i, i = 0..7.  Scales (and zeros) of positions base + n and
// base + 16 + n.  Positions past the split read as 0 (masked later).
template <int MODE>
struct StepData {
  uint4 k[2];
  uint32_t v[8];
  uint16_t ks[2], vs[2], kz[2], vz[2];
};

template <int MODE>
__device__ __forceinline__ void load_step(StepData<MODE>& d, const SplitBuffers& r, int base,
                                          int voff_k, int voff_v, int voff_s) {
  // the step's offset goes into the per-lane offset (the range check covers
  // the per-lane and instruction offsets)
  const int vk = voff_k + base * 64, vv = voff_v + base * 64, vs = voff_s + base * 2;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const auto kk = __builtin_amdgcn_raw_buffer_load_b128(r.k, vk + 1024 * t, 0, 0);
    d.k[t] = make_uint4(kk[0], kk[1], kk[2], kk[3]);
    d.ks[t] = __builtin_amdgcn_raw_buffer_load_b16(r.ks, vs + 32 * t, 0, 0);
    d.vs[t] = __builtin_amdgcn_raw_buffer_load_b16(r.vs, vs + 32 * t, 0, 0);
    if (MODE == 1) {
      d.kz[t] = __builtin_amdgcn_raw_buffer_load_b16(r.kz, vs + 32 * t, 0, 0);
      d.vz[t] = __builtin_amdgcn_raw_buffer_load_b16(r.vz, vs + 32 * t, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    d.v[i] = __builtin_amdgcn_raw_buffer_load_b32(r.v, vv + 256 * i, 0, 0);
}

__device__ __forceinline__ float f16_bits_to_float(uint16_t h) {
  return float(__builtin_bit_cast(_Float16, h));
}

// The online softmax keeps its reference m until a step's maximum exceeds it
// by more than this (log2 units); weights then stay below 2^6.
constexpr float kRescaleSlack = 6.0f;
// Weights are scaled by 2^8 before the fp16 hi / lo split (w * 2^8 < 2^14).
constexpr float kWeightScale = 256.0f;

template <int MODE>
__global__ __launch_bounds__(kDecThreads, 3) void decode_split_kernel(DecodeArgs p) {
  __shared__ float q_rot[kDecHeads][kDecD];
  __shared__ float q_mul[kDecHeads];
  __shared__ __attribute__((aligned(16))) uint32_t wbuf[kDecWaves][16 * 16];
  __shared__ __attribute__((aligned(16))) float cmb_o[kDecWaves][kDecHeads][kDecD];
  __shared__ float cmb_ml[kDecWaves][kDecHeads][2];

  const int bh = blockIdx.x;
  const int split = blockIdx.y;
  const int b = bh / p.hkv, kv = bh - b * p.hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int len = p.max_len;
  if (p.lengths) len = max(0, min(p.lengths[b], p.max_len));
  const int pos_begin = split * p.split_len;
  const int pos_end = min(pos_begin + p.split_len, len);

  // cache buffers over this split's positions [0, pos_end) of the (batch,
  // KV head) rows; lane offsets of the step loads (see load_step)
  const int64_t row0 = (int64_t(b) * p.hkv + kv) * p.s_cache;
  const int nrec = max(pos_end, 0);
  SplitBuffers bufs;
  bufs.k = buffer_of(p.kq + row0 * 64, nrec * 64);
  bufs.v = buffer_of(p.vq + row0 * 64, nrec * 64);
  bufs.ks = buffer_of(p.ks + row0, nrec * 2);
  bufs.vs = buffer_of(p.vs + row0, nrec * 2);
  if (MODE == 1) {
    bufs.kz = buffer_of(p.kz + row0, nrec * 2);
    bufs.vz = buffer_of(p.vz + row0, nrec * 2);
  }
  const int n = lane & 15, g = lane >> 4;  // also (column, row group a) of D
  const int voff_k = n * 64 + 16 * g, voff_v = g * 64 + 4 * n, voff_s = 2 * n;
  int base = pos_begin + kDecStep * wave;
  StepData<MODE> cur;

  // ---- rotate the group's queries: q~ = H_128 diag(s) q / sqrt(128) ------
  {
    const int hh = tid >> 5, c = tid & 31;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (hh < p.group) {
      const __half* src = p.q + (int64_t(b) * p.hq + kv * p.group + hh) * kDecD + 4 * c;
      const uint2 raw = *reinterpret_cast<const uint2*>(src);
      const half2_t h01 = __builtin_bit_cast(half2_t, raw.x);
      const half2_t h23 = __builtin_bit_cast(half2_t, raw.y);
      v[0] = float(h01[0]);
      v[1] = float(h01[1]);
      v[2] = float(h23[0]);
      v[3] = float(h23[1]);
      if (p.signs) {
        const int8_t* sg = p.signs + kv * p.signs_stride_h + 4 * c;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= float(sg[i]);
      }
    }
    // the first step's cache loads go out now, behind the query loads, so
    // their latency overlaps the rotation
    if (base < pos_end) load_step<MODE>(cur, bufs, base, voff_k, voff_v, voff_s);
    // element e = 4 c + i: bits 0, 1 in registers, bits 2 .. 6 across lanes
    const float a0 = v[0] + v[1], a1 = v[0] - v[1], a2 = v[2] + v[3], a3 = v[2] - v[3];
    v[0] = a0 + a2;
    v[2] = a0 - a2;
    v[1] = a1 + a3;
    v[3] = a1 - a3;
#pragma unroll
    for (int k = 1; k < 32; k <<= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float o = __shfl_xor(v[i], k, 32);
        v[i] = (c & k) ? o - v[i] : v[i] + o;
      }
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] *= 0.08838834764831845f;  // 1 / sqrt(128)
      q_rot[hh][4 * c + i] = v[i];
      mx = fmaxf(mx, fabsf(v[i]));
    }
#pragma unroll
    for (int k = 1; k < 32; k <<= 1) mx = fmaxf(mx, __shfl_xor(mx, k, 32));
    if (c == 0) {
      // power of two that brings the head's largest |q~| into [128, 256):
      // the fp16 hi part cannot overflow and the lo part stays normal
      int e = 0;
      (void)frexpf(mx, &e);
      q_mul[hh] = mx > 0.0f ? ldexpf(1.0f, 8 - e) : 1.0f;
    }
  }
  __syncthreads();

  // A operands of the score MFMAs: row m = (head m / 2, hi / lo), k-chunk t
  // covers head dims 32 g + 8 t + perm8(s); x16 slots divided by 16
  half8_t a_q[4];
  {
    const int head = n >> 1;
    const bool lo = n & 1;
    const float qm = q_mul[head];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float x = q_rot[head][32 * g + 8 * t + perm8(s)] * (slot_x16(s) ? qm * 0.0625f : qm);
        const _Float16 hi = _Float16(x);
        a_q[t][s] = lo ? _Float16(x - float(hi)) : hi;
      }
  }
  // per D lane: heads 2 g and 2 g + 1
  float cs[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) cs[hh] = p.score_mul / q_mul[2 * g + hh];


  // fp16 offsets subtracted after the nibble -> fp16 step (see nibbles_to_half8)
  const half2_t v_off1 = MODE == 0 ? half2_t{_Float16(1032.0f), _Float16(1032.0f)}
                                   : half2_t{_Float16(1024.0f), _Float16(1024.0f)};
  const half2_t v_off16 = MODE == 0 ? half2_t{_Float16(1152.0f), _Float16(1152.0f)}
                                    : half2_t{_Float16(1024.0f), _Float16(1024.0f)};
  // weights of positions n and 16 + n sit in x16 slots when (n >> 2) is odd
  const float w_scale = ((n >> 2) & 1) ? kWeightScale * 0.0625f : kWeightScale;

  float m_run[2] = {-1e30f, -1e30f}, l_run[2] = {0.0f, 0.0f}, corr[2] = {0.0f, 0.0f};
  float4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t* wb = wbuf[wave];

  for (; base < pos_end; base += kDecUnit) {
    StepData<MODE> nxt;
    load_step<MODE>(nxt, bufs, base + kDecUnit, voff_k, voff_v, voff_s);

    // ---- scores: D[row][position] over two 16-position tiles --------------
    float4_t sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      half2_t k_off1, k_off16;
      if (MODE == 0) {
        k_off1 = v_off1;
        k_off16 = v_off16;
      } else {
        const float z = f16_bits_to_float(cur.kz[t]);
        const _Float16 z1 = _Float16(1024.0f + z), z16 = _Float16(1024.0f + 16.0f * z);
        k_off1 = half2_t{z1, z1};
        k_off16 = half2_t{z16, z16};
      }
      const uint32_t w[4] = {cur.k[t].x, cur.k[t].y, cur.k[t].z, cur.k[t].w};
      sc[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            a_q[c], nibbles_to_half8<MODE == 0>(w[c], k_off1, k_off16), sc[t], 0, 0, 0);
    }
    // ---- online softmax (log2 domain).  u = score + e(v scale): the
    // weights w = 2^(u - m) * mant(v scale) carry the value scale, while the
    // softmax sum takes 2^(u - m - e) -----------------------------------------
    float u[2][2], vm[2];
    int ve[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      vm[t] = frexpf(f16_bits_to_float(cur.vs[t]), &ve[t]);
      const float ksf = f16_bits_to_float(cur.ks[t]);
      const bool valid = base + 16 * t + n < pos_end;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float s = (sc[t][2 * hh] + sc[t][2 * hh + 1]) * (ksf * cs[hh]);
        u[t][hh] = valid ? s + float(ve[t]) : -INFINITY;
      }
    }
    // the reference m moves only when a step's maximum exceeds it by more
    // than kRescaleSlack; the accumulators are rescaled then
    float alpha[2];
    bool moved = false;
    float mxs[2] = {fmaxf(u[0][0], u[1][0]), fmaxf(u[0][1], u[1][1])};
    row_max16x2(mxs[0], mxs[1]);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float mx = mxs[hh];
      alpha[hh] = 1.0f;
      if (mx > m_run[hh] + kRescaleSlack) {
        alpha[hh] = __builtin_amdgcn_exp2f(m_run[hh] - mx);
        m_run[hh] = mx;
        moved = true;
      }
    }
    float wt[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float lsum = 0.0f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float ex = __builtin_amdgcn_exp2f(u[t][hh] - m_run[hh]);
        wt[t][hh] = ex * vm[t];
        lsum += ldexpf(ex, -ve[t]);
      }
      l_run[hh] = l_run[hh] * alpha[hh] + lsum;
      if (MODE == 1)
        corr[hh] = corr[hh] * alpha[hh] + wt[0][hh] * f16_bits_to_float(cur.vz[0]) +
                   wt[1][hh] * f16_bits_to_float(cur.vz[1]);
    }
    // ---- weights to LDS in the A layout of the P V MFMAs ------------------
    // row 4 g + 2 hh (+1 for lo), k-slot of position q: group q & 3, slot
    // inverse-perm8(q >> 2); positions n and 16 + n share one dword
    {
      const int off = (n & 3) * 4 + (n >> 2);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float w0 = wt[0][hh] * w_scale, w1 = wt[1][hh] * w_scale;
        const _Float16 h0 = _Float16(w0), h1 = _Float16(w1);
        const _Float16 l0 = _Float16(w0 - float(h0)), l1 = _Float16(w1 - float(h1));
        const int row = 4 * g + 2 * hh;
        wb[row * 16 + off] = __builtin_bit_cast(uint32_t, half2_t{h0, h1});
        wb[(row + 1) * 16 + off] = __builtin_bit_cast(uint32_t, half2_t{l0, l1});
      }
    }
    if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[j][0] *= alpha[0];
        acc[j][1] *= alpha[0];
        acc[j][2] *= alpha[1];
        acc[j][3] *= alpha[1];
      }
    }
    const half8_t a_w = *reinterpret_cast<const half8_t*>(&wb[n * 16 + g * 4]);
    // ---- P V: V nibbles transposed to (dim, 8 positions) per register -----
    uint32_t r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = cur.v[i];
    transpose_nibbles8(r);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          a_w, nibbles_to_half8<MODE == 0>(r[j], v_off1, v_off16), acc[j], 0, 0, 0);
    cur = nxt;
  }

  // ---- merge the four waves, write the split's partial result -------------
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    l_run[hh] = row_sum16(l_run[hh]);
    if (MODE == 1) corr[hh] = row_sum16(corr[hh]);
    const int head = 2 * g + hh;
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      o[j] = (acc[j][2 * hh] + acc[j][2 * hh + 1]) * (1.0f / kWeightScale) - corr[hh];
    float4* dst = reinterpret_cast<float4*>(&cmb_o[wave][head][8 * n]);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
    if (n == 0) {
      cmb_ml[wave][head][0] = m_run[hh];
      cmb_ml[wave][head][1] = l_run[hh];
    }
  }
  __syncthreads();
  {
    const int head = tid >> 5, c = tid & 31;
    if (head < p.group) {
      float mw[kDecWaves], big = -INFINITY;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        mw[w] = cmb_ml[w][head][0];
        big = fmaxf(big, mw[w]);
      }
      float lsum = 0.0f;
      float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(mw[w] - big);
        lsum += f * cmb_ml[w][head][1];
        const float4 x = reinterpret_cast<const float4*>(cmb_o[w][head])[c];
        o.x += f * x.x;
        o.y += f * x.y;
        o.z += f * x.z;
        o.w += f * x.w;
      }
      const int64_t slot = (int64_t(bh) * p.splits + split) * p.group + head;
      reinterpret_cast<float4*>(p.part_o + slot * kDecD)[c] = o;
      if (c == 0) {
        p.part_ml[2 * slot] = big;
        p.part_ml[2 * slot + 1] = lsum;
      }
    }
  }
}

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  int hkv, hq, group, splits;
  __half* out;     // [B, Hq, 128]
  float* out_f32;  // optional, same layout
};

constexpr int kCombineBatch = 8;  // split partials loaded together
constexpr int kCombineDims = 4;   // head dims per combine block

// Block (b, kCombineDims-dim chunk): every query head's outputs in the
// chunk, one per thread.  Each thread merges its head's splits (loads issued
// kCombineBatch at a time, so a few memory round trips cover all splits).
// With CROSS the Walsh-Hadamard transform over the head index (Sylvester
// order, normalised by 1 / sqrt(Hq)) runs on lane shuffles for up to 64
// query heads and in LDS, a barrier per stage, for 128 and 256 heads (the
// dynamic LDS is allocated only then).
template <bool CROSS>
__global__ __launch_bounds__(1024) void decode_combine_kernel(CombineArgs p) {
  extern __shared__ float zs[];  // [Hq][kCombineDims]
  constexpr int W = kCombineDims;
  const int b = blockIdx.x, d0 = W * blockIdx.y;
  const int total = p.hq * W;
  // With at most 64 query heads, thread idx takes head idx % Hq and dim
  // idx / Hq: the heads of one dim sit on the lanes of one wave, and the
  // transform over the head index is a chain of lane shuffles (no LDS, no
  // barriers).  Every thread then runs exactly one iteration (blockDim.x is
  // total), and partner lanes idx ^ h (h < Hq) are threads of the block.
  const bool on_lanes = CROSS && p.hq <= 64;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int hq = on_lanes ? (idx & (p.hq - 1)) : idx / W;
    const int dl = on_lanes ? (idx / p.hq) : idx % W;
    const int kv = hq / p.group, gi = hq - kv * p.group;
    const int64_t s0 = (int64_t(b) * p.hkv + kv) * p.splits;
    float big = -INFINITY, lsum = 0.0f, o = 0.0f;
    for (int sb = 0; sb < p.splits; sb += kCombineBatch) {
      float mv[kCombineBatch], lv[kCombineBatch], ov[kCombineBatch];
#pragma unroll
      for (int i = 0; i < kCombineBatch; ++i) {
        mv[i] = -INFINITY;
        lv[i] = 0.0f;
        ov[i] = 0.0f;
        if (sb + i < p.splits) {
          const int64_t slot = (s0 + sb + i) * p.group + gi;
          mv[i] = p.part_ml[2 * slot];
          lv[i] = p.part_ml[2 * slot + 1];
          ov[i] = p.part_o[slot * kDecD + d0 + dl];
        }
      }
      float nb = big;
#pragma unroll
      for (int i = 0; i < kCombineBatch; ++i) nb = fmaxf(nb, mv[i]);
      const float f0 = __builtin_amdgcn_exp2f(big - nb);
      lsum *= f0;
      o *= f0;
#pragma unroll
      for (int i = 0; i < kCombineBatch; ++i) {
        const float f = __builtin_amdgcn_exp2f(mv[i] - nb);
        lsum += f * lv[i];
        o += f * ov[i];
      }
      big = nb;
    }
    const float res = lsum > 0.0f ? o / lsum : 0.0f;
    if (CROSS && on_lanes) {
      float v = res;
      for (int h = 1; h < p.hq; h <<= 1) {
        const float w = __shfl_xor(v, h);
        v = (hq & h) ? w - v : v + w;
      }
      v *= 1.0f / sqrtf(float(p.hq));
      const int64_t at = (int64_t(b) * p.hq + hq) * kDecD + d0 + dl;
      p.out[at] = __float2half_rn(v);
      if (p.out_f32) p.out_f32[at] = v;
    } else if (CROSS) {
      zs[idx] = res;
    } else {
      const int64_t at = (int64_t(b) * p.hq + hq) * kDecD + d0 + dl;
      p.out[at] = __float2half_rn(res);
      if (p.out_f32) p.out_f32[at] = res;
    }
  }
  if (!CROSS || on_lanes) return;
  __syncthreads();
  const int half_total = total / 2;
  for (int h = 1; h < p.hq; h <<= 1) {
    for (int idx = threadIdx.x; idx < half_total; idx += blockDim.x) {
      const int i = idx / W, dl = idx % W;
      const int lo = (i / h) * 2 * h + (i % h), hi = lo + h;
      const float a = zs[lo * W + dl], c = zs[hi * W + dl];
      zs[lo * W + dl] = a + c;
      zs[hi * W + dl] = a - c;
    }
    __syncthreads();
  }
  const float norm = 1.0f / sqrtf(float(p.hq));
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int hq = idx / W, dl = idx % W;
    const float res = zs[idx] * norm;
    const int64_t at = (int64_t(b) * p.hq + hq) * kDecD + d0 + dl;
    p.out[at] = __float2half_rn(res);
    if (p.out_f32) p.out_f32[at] = res;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: the per-split partials live in
// a file-scope device array of QUAROT_DECODE_SCRATCH_BYTES (each GPU the
// library runs on holds its own copy until the process ends).  Host code
// never passes the array's name to a kernel: its device address is fetched
// once per device with hipGetSymbolAddress, with that device current, and
// kept per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[QUAROT_DECODE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

int decode_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("hipGetDevice: %s", hipGetErrorString(e));
    return QUAROT_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device %d: the allocation-free entry point serves devices 0..%d", dev,
              kMaxDevices - 1);
    return QUAROT_ERR_UNSUPPORTED;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) {
        set_error("hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        return QUAROT_ERR_HIP;
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return QUAROT_OK;
}

// Split workgroups planned per round on MI355X: 256 CUs x 2.  The kernel's
// register use would allow four 4-wave groups per CU, but two (two waves per
// SIMD) already keep the step loop at the VALU's rate, while every further
// group adds its dispatch, its query rotation and its partials to merge
// (70B shape: 4 splits of 1024 positions ran 23.1 us against 24.7 us for 8
// splits of 512).
constexpr int64_t kDecResident = 512;

void decode_plan(int64_t B, int64_t Hkv, int64_t max_len, int& splits, int& split_len) {
  // Choose the split count that minimises (rounds of resident workgroups) x
  // (steps per wave + one step's worth of per-group overhead); ties go to
  // fewer splits (less partial traffic).  Splits are whole 32-position steps.
  const int64_t steps = (max_len + kDecStep - 1) / kDecStep;
  const int64_t pairs = B * Hkv;
  int64_t best = 1, best_cost = -1;
  for (int64_t s = 1; s <= steps && s <= 256; ++s) {
    const int64_t per = (steps + s - 1) / s;
    const int64_t rounds = (pairs * s + kDecResident - 1) / kDecResident;
    const int64_t cost = rounds * ((per + kDecWaves - 1) / kDecWaves + 1);
    if (best_cost < 0 || cost < best_cost) {
      best = s;
      best_cost = cost;
    }
  }
  const int64_t per = (steps + best - 1) / best;
  splits = int((steps + per - 1) / per);
  split_len = int(per * kDecStep);
}

int64_t decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_len) {
  int splits = 0, split_len = 0;
  decode_plan(B, Hkv, max_len, splits, split_len);
  const int64_t slots = B * Hkv * splits * (Hq / Hkv);
  return slots * (kDecD + 2) * int64_t(sizeof(float));
}

int launch_kv_decode(const DecodeTensors& t, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t S_cache, int64_t max_len, float sm_scale, int mode, bool cross,
                     hipStream_t stream) {
  DecodeArgs p{};
  p.q = t.q;
  p.signs = t.signs;
  p.signs_stride_h = t.signs_stride_h;
  p.kq = t.k_q;
  p.ks = t.k_scale;
  p.kz = t.k_zero;
  p.vq = t.v_q;
  p.vs = t.v_scale;
  p.vz = t.v_zero;
  p.hkv = int(Hkv);
  p.hq = int(Hq);
  p.group = int(Hq / Hkv);
  p.s_cache = S_cache;
  p.max_len = int(max_len);
  p.lengths = t.lengths;
  decode_plan(B, Hkv, max_len, p.splits, p.split_len);
  p.score_mul = sm_scale * 1.4426950408889634f;
  const int64_t slots = B * Hkv * p.splits * p.group;
  p.part_o = static_cast<float*>(t.workspace);
  p.part_ml = p.part_o + slots * kDecD;

  const dim3 grid{unsigned(B * Hkv), unsigned(p.splits)}, block{unsigned(kDecThreads)};
  if (mode == 1)
    hipLaunchKernelGGL(decode_split_kernel<1>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(decode_split_kernel<0>, grid, block, 0, stream, p);
  int st = check_launch("kv_decode split");
  if (st != QUAROT_OK) return st;

  CombineArgs c{p.part_o, p.part_ml, p.hkv, p.hq, p.group, p.splits, t.out, t.out_f32};
  const dim3 cgrid{unsigned(B), unsigned(kDecD / kCombineDims)};
  const unsigned cthreads = unsigned(std::min<int64_t>(Hq * kCombineDims, 1024));
  // LDS only for the transform of more than 64 heads (the lane path uses none)
  const size_t lds = (cross && Hq > 64) ? size_t(Hq) * kCombineDims * sizeof(float) : 0;
  if (cross)
    hipLaunchKernelGGL(decode_combine_kernel<true>, cgrid, dim3(cthreads), lds, stream, c);
  else
    hipLaunchKernelGGL(decode_combine_kernel<false>, cgrid, dim3(cthreads), 0, stream, c);
  return check_launch("kv_decode combine");
}

}  // namespace quarot
