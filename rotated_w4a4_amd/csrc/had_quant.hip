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
//   * had_quant_4096_split  d = 4096: two waves per row, one LDS exchange
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

template <int D, bool CLAMP, bool RMS>
__global__ __launch_bounds__(kQuadBlock) void had_quant_quad(
    const __half* __restrict__ x, int64_t rows, int64_t ld_x, const int8_t* __restrict__ signs,
    float clip_ratio, uint8_t* __restrict__ q_out, int64_t ld_q, __half* __restrict__ scale_out,
    float* __restrict__ x_rot, float rms_eps) {
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
    quad_row<D, CLAMP, RMS>(raw, q_out + rr * ld_q, scale_out + rr,
                            x_rot ? x_rot + rr * D : nullptr, mask, lane_q, clip_ratio, active,
                            rms_eps);
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

template <int M, bool RMS>
__global__ __launch_bounds__(kLdsBlock) void had_quant_lds(
    const __half* __restrict__ x, int64_t rows, int d, int n, int64_t ld_x,
    const int8_t* __restrict__ signs, float clip_ratio, uint8_t* __restrict__ q_out, int64_t ld_q,
    __half* __restrict__ scale_out, float* __restrict__ x_rot, float norm, float rms_eps) {
  extern __shared__ float buf[];
  __shared__ float red[kLdsBlock / 64];
  __shared__ float red_ss[kLdsBlock / 64];
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
    float amax = 0.0f, ss = 0.0f;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float y = buf[pidx(8 * c + i)] * norm;
        amax = fmaxf(amax, fabsf(y));
        if (RMS) ss = fmaf(y, y, ss);
      }
    }
    amax = wave_max(amax);
    if (RMS) ss = wave_sum_dpp(ss);
    if ((threadIdx.x & 63) == 0) {
      red[threadIdx.x >> 6] = amax;
      if (RMS) red_ss[threadIdx.x >> 6] = ss;
    }
    __syncthreads();
    amax = red[0];
    for (int w = 1; w < int(blockDim.x >> 6); ++w) amax = fmaxf(amax, red[w]);
    // RMS: normalise by 1 / sqrt(mean(x^2) + eps); the rotation keeps the norm
    float rs = 1.0f;
    if (RMS) {
      float tot = 0.0f;
      for (int w = 0; w < int(blockDim.x >> 6); ++w) tot += red_ss[w];
      rs = rsqrtf(tot / float(d) + rms_eps);
    }
    const __half s16 = row_scale_fp16(amax * rs, clip_ratio);
    const float k = inv_scale(s16);
    // 5. quantise, pack, store
    uint8_t* qrow = q_out + row * ld_q;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
      float f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = buf[pidx(8 * c + i)] * (norm * rs);
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
                     __half* scale_out, float* x_rot_out, float rms_eps, hipStream_t stream) {
  const int cus = sm_count_cached();
  const bool rms = rms_eps >= 0.0f;  // normalise each row by its RMS first
  const bool clamp = clip_ratio != 1.0f;
  if (m == 1 && d <= 256) {
    const int64_t rpb = kQuadBlock / 4;
    int64_t blocks = (rows + rpb - 1) / rpb;
    // at most 2^16 blocks (beyond, blocks loop), far below the 2^32
    // work-item limit of a grid dimension
    const int64_t cap = int64_t(1) << 16;
    if (blocks > cap) blocks = cap;
    const dim3 grid{unsigned(blocks)}, block{unsigned(kQuadBlock)};
#define QR_QUAD(DD, CL, RM)                                                                    \
  hipLaunchKernelGGL((had_quant_quad<DD, CL, RM>), grid, block, 0, stream, x, rows, ld_x, signs, \
                     clip_ratio, q_out, ld_q, scale_out, x_rot_out, rms_eps)
#define QR_QUAD_D(DD)                   \
  if (rms) {                            \
    if (clamp) QR_QUAD(DD, true, true); \
    else QR_QUAD(DD, false, true);      \
  } else {                              \
    if (clamp) QR_QUAD(DD, true, false); \
    else QR_QUAD(DD, false, false);     \
  }
    switch (d) {
      case 32: QR_QUAD_D(32); break;
      case 64: QR_QUAD_D(64); break;
      case 128: QR_QUAD_D(128); break;
      default: QR_QUAD_D(256); break;
    }
#undef QR_QUAD_D
#undef QR_QUAD
    return check_launch("had_quant_quad");
  }
  if (m == 1 && d == 4096) {
    const int64_t cap = int64_t(cus) * 8;  // 16 KiB LDS, two waves per block
    const int64_t blocks = rows < cap ? rows : cap;
    const dim3 grid{unsigned(blocks)}, block{unsigned(kSplitBlock)};
#define QR_SPLIT(CL, RM)                                                                       \
  hipLaunchKernelGGL((had_quant_4096_split<CL, RM>), grid, block, 0, stream, x, rows, ld_x, signs, \
                     clip_ratio, q_out, ld_q, scale_out, x_rot_out, rms_eps)
    if (rms) {
      if (clamp) QR_SPLIT(true, true); else QR_SPLIT(false, true);
    } else {
      if (clamp) QR_SPLIT(true, false); else QR_SPLIT(false, false);
    }
#undef QR_SPLIT
    return check_launch("had_quant_4096_split");
  }
  if ((m == 12 || m == 28) && d == 1024 * m) {
    static const bool kron_attr_ok = [] {
      bool ok = true;
#define QR_ATTR(MM, CL, RM)                                                                  \
  ok &= hipFuncSetAttribute(reinterpret_cast<const void*>(had_quant_kron<MM, CL, RM>),       \
                            hipFuncAttributeMaxDynamicSharedMemorySize,                      \
                            KronCfg<MM>::LDS_BYTES) == hipSuccess
      QR_ATTR(12, false, false);
      QR_ATTR(12, true, false);
      QR_ATTR(12, false, true);
      QR_ATTR(12, true, true);
      QR_ATTR(28, false, false);
      QR_ATTR(28, true, false);
      QR_ATTR(28, false, true);
      QR_ATTR(28, true, true);
#undef QR_ATTR
      return ok;
    }();
    if (!kron_attr_ok) {
      set_error("could not raise the dynamic LDS limit for d = %d", d);
      return QUAROT_ERR_HIP;
    }
    const size_t lds = m == 12 ? KronCfg<12>::LDS_BYTES : KronCfg<28>::LDS_BYTES;
    // two waves per SIMD (up to 256 VGPRs): two 256-thread blocks per CU for
    // m = 12, one 512-thread block for m = 28
    const int64_t cap =
        int64_t(cus) * (m == 12 ? KronCfg<12>::BLOCKS_PER_CU : KronCfg<28>::BLOCKS_PER_CU);
    const int64_t blocks = rows < cap ? rows : cap;
    const unsigned threads = m == 12 ? KronCfg<12>::THREADS : KronCfg<28>::THREADS;
    const dim3 grid{unsigned(blocks)}, block{threads};
    const float norm = 1.0f / sqrtf(float(d));
#define QR_KRON(MM, CL, RM)                                                                     \
  hipLaunchKernelGGL((had_quant_kron<MM, CL, RM>), grid, block, lds, stream, x, rows, ld_x, signs, \
                     clip_ratio, q_out, ld_q, scale_out, x_rot_out, norm, rms_eps)
#define QR_KRON_M(MM)                    \
  if (rms) {                             \
    if (clamp) QR_KRON(MM, true, true);  \
    else QR_KRON(MM, false, true);       \
  } else {                               \
    if (clamp) QR_KRON(MM, true, false); \
    else QR_KRON(MM, false, false);      \
  }
    if (m == 12) {
      QR_KRON_M(12);
    } else {
      QR_KRON_M(28);
    }
#undef QR_KRON_M
#undef QR_KRON
    return check_launch("had_quant_kron");
  }
  const size_t lds = size_t(d + d / 32) * sizeof(float);
  // the generic kernel stages up to 32768 + 1024 floats (132 KiB) in LDS
  static const bool lds_attr_ok = [] {
    const int bytes = (32768 + 1024) * int(sizeof(float));
    bool ok = true;
#define QR_ATTR(MM, RM)                                                                       \
  ok &= hipFuncSetAttribute(reinterpret_cast<const void*>(had_quant_lds<MM, RM>),             \
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess
    QR_ATTR(1, false);
    QR_ATTR(12, false);
    QR_ATTR(28, false);
    QR_ATTR(1, true);
    QR_ATTR(12, true);
    QR_ATTR(28, true);
#undef QR_ATTR
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
#define QR_LDS(MM, RM)                                                                         \
  hipLaunchKernelGGL((had_quant_lds<MM, RM>), grid, block, lds, stream, x, rows, d, n, ld_x,   \
                     signs, clip_ratio, q_out, ld_q, scale_out, x_rot_out, norm, rms_eps)
  switch (m) {
    case 1:
      if (rms) QR_LDS(1, true); else QR_LDS(1, false);
      break;
    case 12:
      if (rms) QR_LDS(12, true); else QR_LDS(12, false);
      break;
    default:
      if (rms) QR_LDS(28, true); else QR_LDS(28, false);
      break;
  }
#undef QR_LDS
  return check_launch("had_quant_lds");
}

}  // namespace quarot
