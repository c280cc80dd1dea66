// quarot_had_quant kernels: fused randomized Hadamard rotation + per-token
// symmetric INT4 quantisation with nibble packing.
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary): section 3.4 Stage 1a (R = H diag(s); H_d = H_{2^n} (x) H_m for
// d = 2^n m), Stage 1b (online FWHT in FP32 before the down-projection),
// Stage 2b (per-token symmetric scale) and "Kernel Implementation and
// Hardware Efficiency" (quantise, pack two INT4 per byte).  "QuaRot Guide",
// section 3 of "The Architecture": the FWHT is d log d additions and
// subtractions.
//
// Kernels:
//   * had_quant_quad<D>   d = 32..256: a quad of lanes per row (quad_rows.h).
//   * had_quant_4096_split  d = 4096: four waves per row, one LDS exchange
//                         (split_rows.h).
//   * had_quant_kron<M>   d = 1024 m, m = 12 or 28: a workgroup per row, H_m
//                         on the matrix cores, one LDS exchange (kron_rows.h).
//   * had_quant_lds<M>    any supported d (<= 32768): one workgroup per row,
//                         the row staged in LDS as fp32; H_m applied per
//                         contiguous group, then radix-32 FWHT passes over
//                         the power-of-two index.
#include "quad_rows.h"
#include "wave_rows.h"
#include "kron_rows.h"
#include "split_rows.h"

namespace quarot {

namespace {

constexpr int kQuadBlock = 256;  // 64 rows per block iteration

template <int D, bool CLAMP>
__global__ __launch_bounds__(kQuadBlock) void had_quant_quad(
    const __half* __restrict__ x, int64_t rows, int64_t ld_x, const int8_t* __restrict__ signs,
    float clip_ratio, uint8_t* __restrict__ q_out, int64_t ld_q, __half* __restrict__ scale_out,
    float* __restrict__ x_rot) {
  constexpr int NC = D / 32;
  const int lane_q = threadIdx.x & 3;
  uint4 mask[NC];
  load_sign_masks<NC>(signs, lane_q, mask);
  const int64_t rows_per_block = kQuadBlock / 4;
  const int64_t step = int64_t(gridDim.x) * rows_per_block;
  // the grid normally covers every row once; the loop serves capped grids
  for (int64_t base = int64_t(blockIdx.x) * rows_per_block; base < rows; base += step) {
    const int64_t r = base + (threadIdx.x >> 2);
    const bool active = r < rows;
    const int64_t rr = active ? r : 0;
    uint4 raw[NC];
    quad_load<D>(x + rr * ld_x, lane_q, raw);
    quad_row<D, CLAMP>(raw, q_out + rr * ld_q, scale_out + rr, x_rot ? x_rot + rr * D : nullptr,
                       mask, lane_q, clip_ratio, active);
  }
}

// ---------------------------------------------------------------------------
// Generic path: one workgroup per row, fp32 row in LDS.
// ---------------------------------------------------------------------------
constexpr int kLdsBlock = 512;
constexpr int kRadixBits = 5;  // 32 values per FWHT task

// LDS index with one pad word per 32 to spread strided accesses over banks.
__device__ __forceinline__ int pidx(int e) { return e + (e >> 5); }

template <int M>
__device__ __forceinline__ void apply_hm(float* buf, int d) {
  constexpr HadFactor<M> H = HadTable<M>::value;
  const int groups = d / M;
  for (int g = threadIdx.x; g < groups; g += blockDim.x) {
    float in[M], out[M];
#pragma unroll
    for (int b = 0; b < M; ++b) in[b] = buf[pidx(g * M + b)];
#pragma unroll
    for (int b = 0; b < M; ++b) {
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < M; ++c) acc = (H.v[b][c] > 0) ? acc + in[c] : acc - in[c];
      out[b] = acc;
    }
#pragma unroll
    for (int b = 0; b < M; ++b) buf[pidx(g * M + b)] = out[b];
  }
}

// One radix-2^R pass of the FWHT over the power-of-two index a (stride M)
// covering index bits [s, s + R).
template <int R, int M>
__device__ __forceinline__ void fwht_pass(float* buf, int n, int s) {
  const int tasks = (M << n) >> R;
  for (int t = threadIdx.x; t < tasks; t += blockDim.x) {
    const int b = t % M;
    const int rest = t / M;
    const int lo = rest & ((1 << s) - 1);
    const int hi = rest >> s;
    const int a0 = lo | (hi << (s + R));
    float v[1 << R];
#pragma unroll
    for (int j = 0; j < (1 << R); ++j) v[j] = buf[pidx((a0 + (j << s)) * M + b)];
#pragma unroll
    for (int h = 1; h < (1 << R); h <<= 1) {
#pragma unroll
      for (int j = 0; j < (1 << R); ++j) {
        if ((j & h) == 0) {
          const float p = v[j], q = v[j + h];
          v[j] = p + q;
          v[j + h] = p - q;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < (1 << R); ++j) buf[pidx((a0 + (j << s)) * M + b)] = v[j];
  }
}

template <int M>
__global__ __launch_bounds__(kLdsBlock) void had_quant_lds(
    const __half* __restrict__ x, int64_t rows, int d, int n, int64_t ld_x,
    const int8_t* __restrict__ signs, float clip_ratio, uint8_t* __restrict__ q_out, int64_t ld_q,
    __half* __restrict__ scale_out, float* __restrict__ x_rot, float norm) {
  extern __shared__ float buf[];
  __shared__ float red[kLdsBlock / 64];
  const int chunks = d / 8;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const __half* src = x + row * ld_x;
    // 1. load, flip signs, widen to fp32
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
      const uint4 raw = *reinterpret_cast<const uint4*>(src + 8 * c);
      float f[8];
      unpack_half8(raw, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float sgn = (signs && signs[8 * c + i] < 0) ? -1.0f : 1.0f;
        buf[pidx(8 * c + i)] = f[i] * sgn;
      }
    }
    __syncthreads();
    // 2. H_m on each contiguous group of m
    if (M > 1) {
      apply_hm<M>(buf, d);
      __syncthreads();
    }
    // 3. FWHT over the 2^n index, radix-32 passes (last pass may be smaller)
    int s = 0;
    while (s < n) {
      const int r = (n - s >= kRadixBits) ? kRadixBits : (n - s);
      switch (r) {
        case 5: fwht_pass<5, M>(buf, n, s); break;
        case 4: fwht_pass<4, M>(buf, n, s); break;
        case 3: fwht_pass<3, M>(buf, n, s); break;
        case 2: fwht_pass<2, M>(buf, n, s); break;
        default: fwht_pass<1, M>(buf, n, s); break;
      }
      s += r;
      __syncthreads();
    }
    // 4. row absmax
    float amax = 0.0f;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(buf[pidx(8 * c + i)] * norm));
    }
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = red[0];
    for (int w = 1; w < int(blockDim.x >> 6); ++w) amax = fmaxf(amax, red[w]);
    const __half s16 = row_scale_fp16(amax, clip_ratio);
    const float k = inv_scale(s16);
    // 5. quantise, pack, store
    uint8_t* qrow = q_out + row * ld_q;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
      float f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = buf[pidx(8 * c + i)] * norm;
      *reinterpret_cast<uint32_t*>(qrow + 4 * c) = pack8(f, k);
      if (x_rot) {
        float4* dst = reinterpret_cast<float4*>(x_rot + row * int64_t(d) + 8 * c);
        dst[0] = make_float4(f[0], f[1], f[2], f[3]);
        dst[1] = make_float4(f[4], f[5], f[6], f[7]);
      }
    }
    if (threadIdx.x == 0) scale_out[row] = s16;
    __syncthreads();  // buf and red are reused by the next row
  }
}

int sm_count_cached() {
  static int count = [] {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 256;
    return c > 0 ? c : 256;
  }();
  return count;
}

}  // namespace

int launch_had_quant(const __half* x, int64_t rows, int d, int n, int m, int64_t ld_x,
                     const int8_t* signs, float clip_ratio, uint8_t* q_out, int64_t ld_q,
                     __half* scale_out, float* x_rot_out, hipStream_t stream) {
  const int cus = sm_count_cached();
  if (m == 1 && d <= 256) {
    const int64_t rpb = kQuadBlock / 4;
    int64_t blocks = (rows + rpb - 1) / rpb;
    const int64_t cap = int64_t(1) << 24;  // grid limit; beyond it blocks loop
    if (blocks > cap) blocks = cap;
    const dim3 grid{unsigned(blocks)}, block{unsigned(kQuadBlock)};
#define QR_QUAD(DD, CL)                                                                 \
  hipLaunchKernelGGL((had_quant_quad<DD, CL>), grid, block, 0, stream, x, rows, ld_x, signs, \
                     clip_ratio, q_out, ld_q, scale_out, x_rot_out)
    const bool clamp = clip_ratio != 1.0f;
    switch (d) {
      case 32: if (clamp) QR_QUAD(32, true); else QR_QUAD(32, false); break;
      case 64: if (clamp) QR_QUAD(64, true); else QR_QUAD(64, false); break;
      case 128: if (clamp) QR_QUAD(128, true); else QR_QUAD(128, false); break;
      default: if (clamp) QR_QUAD(256, true); else QR_QUAD(256, false); break;
    }
#undef QR_QUAD
    return check_launch("had_quant_quad");
  }
  if (m == 1 && d == 4096) {
    const int64_t cap = int64_t(cus) * 8;  // 16 KiB LDS, two waves per block
    const int64_t blocks = rows < cap ? rows : cap;
    const dim3 grid{unsigned(blocks)}, block{unsigned(kSplitBlock)};
    if (clip_ratio == 1.0f)
      hipLaunchKernelGGL(had_quant_4096_split<false>, grid, block, 0, stream, x, rows, ld_x, signs,
                         clip_ratio, q_out, ld_q, scale_out, x_rot_out);
    else
      hipLaunchKernelGGL(had_quant_4096_split<true>, grid, block, 0, stream, x, rows, ld_x, signs,
                         clip_ratio, q_out, ld_q, scale_out, x_rot_out);
    return check_launch("had_quant_4096_split");
  }
  if ((m == 12 || m == 28) && d == 1024 * m) {
    static const bool kron_attr_ok = [] {
      bool ok = true;
      ok &= hipFuncSetAttribute(reinterpret_cast<const void*>(had_quant_kron<12, false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                KronCfg<12>::LDS_BYTES) == hipSuccess;
      ok &= hipFuncSetAttribute(reinterpret_cast<const void*>(had_quant_kron<12, true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                KronCfg<12>::LDS_BYTES) == hipSuccess;
      ok &= hipFuncSetAttribute(reinterpret_cast<const void*>(had_quant_kron<28, false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                KronCfg<28>::LDS_BYTES) == hipSuccess;
      ok &= hipFuncSetAttribute(reinterpret_cast<const void*>(had_quant_kron<28, true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                KronCfg<28>::LDS_BYTES) == hipSuccess;
      return ok;
    }();
    if (!kron_attr_ok) {
      set_error("could not raise the dynamic LDS limit for d = %d", d);
      return QUAROT_ERR_HIP;
    }
    const size_t lds = m == 12 ? KronCfg<12>::LDS_BYTES : KronCfg<28>::LDS_BYTES;
    const int64_t cap = cus;  // about 210-255 VGPRs: one 512-thread block per CU
    const int64_t blocks = rows < cap ? rows : cap;
    const dim3 grid{unsigned(blocks)}, block{unsigned(kKronBlock)};
    const float norm = 1.0f / sqrtf(float(d));
    const bool clamp = clip_ratio != 1.0f;
#define QR_KRON(MM, CL)                                                                      \
  hipLaunchKernelGGL((had_quant_kron<MM, CL>), grid, block, lds, stream, x, rows, ld_x, signs, \
                     clip_ratio, q_out, ld_q, scale_out, x_rot_out, norm)
    if (m == 12) {
      if (clamp) QR_KRON(12, true); else QR_KRON(12, false);
    } else {
      if (clamp) QR_KRON(28, true); else QR_KRON(28, false);
    }
#undef QR_KRON
    return check_launch("had_quant_kron");
  }
  const size_t lds = size_t(d + d / 32) * sizeof(float);
  // rows above 16K elements need more than the default 64 KiB of dynamic LDS
  static const bool lds_attr_ok = [] {
    const int bytes = (32768 + 1024) * int(sizeof(float));
    bool ok = true;
    ok &= hipFuncSetAttribute(reinterpret_cast<const void*>(had_quant_lds<1>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess;
    ok &= hipFuncSetAttribute(reinterpret_cast<const void*>(had_quant_lds<12>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess;
    ok &= hipFuncSetAttribute(reinterpret_cast<const void*>(had_quant_lds<28>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess;
    return ok;
  }();
  if (!lds_attr_ok && lds > 65536) {
    set_error("could not raise the dynamic LDS limit for d = %d", d);
    return QUAROT_ERR_HIP;
  }
  const int64_t per_cu = (lds <= 40 * 1024) ? 4 : (lds <= 76 * 1024 ? 2 : 1);
  int64_t blocks = rows < int64_t(cus) * per_cu ? rows : int64_t(cus) * per_cu;
  const dim3 grid{unsigned(blocks)}, block{unsigned(kLdsBlock)};
  const float norm = 1.0f / sqrtf(float(d));
  switch (m) {
    case 1:
      hipLaunchKernelGGL(had_quant_lds<1>, grid, block, lds, stream, x, rows, d, n, ld_x, signs, clip_ratio, q_out, ld_q, scale_out, x_rot_out, norm);
      break;
    case 12:
      hipLaunchKernelGGL(had_quant_lds<12>, grid, block, lds, stream, x, rows, d, n, ld_x, signs, clip_ratio, q_out, ld_q, scale_out, x_rot_out, norm);
      break;
    default:
      hipLaunchKernelGGL(had_quant_lds<28>, grid, block, lds, stream, x, rows, d, n, ld_x, signs, clip_ratio, q_out, ld_q, scale_out, x_rot_out, norm);
      break;
  }
  return check_launch("had_quant_lds");
}

}  // namespace quarot
