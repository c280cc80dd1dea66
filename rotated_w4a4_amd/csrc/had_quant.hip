// quarot_had_quant / quarot_swiglu_had_quant kernels: fused randomized
// Hadamard rotation + per-token symmetric INT4 quantisation with nibble
// packing.
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary): section 3.4 Stage 1a (R = H diag(s); H_d = H_{2^n} (x) H_m for
// d = 2^n m), Stage 1b (online FWHT in FP32 before the down-projection, on
// the SwiGLU product), Stage 2b (per-token symmetric scale) and "Kernel
// Implementation and Hardware Efficiency" (quantise, pack two INT4 per
// byte).  "QuaRot Guide", section 3 of "The Architecture": the FWHT is
// d log d additions and subtractions.
//
// Kernels:
//   * had_quant_quad<D>   d = 32..256, m = 1: a quad of lanes per row
//                         (quad_rows.h).
//   * had_quant_4096_split  d = 4096, m = 1: two waves per row, one LDS
//                         exchange (split_rows.h).
//   * had_quant_kront<M>  d = 12288, plain rows: a workgroup per row, H_2 (x)
//                         H_12 over 512 groups of 24 on the matrix cores,
//                         every butterfly in registers, one b-major LDS
//                         exchange (kront_rows.h).
//   * had_quant_kron<M>   d = 1024 m, m = 12 or 28, for d = 28672 and the
//                         gated product: DPP butterflies over lane bits, one
//                         LDS exchange (kron_rows.h).
//   * had_quant_lds       any supported d (<= 32768) and m: one workgroup per
//                         row, the row staged in LDS as fp32; H_m applied per
//                         contiguous group, then radix-32 FWHT passes over
//                         the power-of-two index; also the gated product.
#include "quad_rows.h"
#include "wave_rows.h"
#include "kron_rows.h"
#include "kront_rows.h"
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

// H_m on every contiguous group of m (m <= 32), entries from the masks:
// y[b] = sum_c (+-1) x[c], the sign from bit c of neg[b].
__device__ __forceinline__ void apply_hm(float* buf, int d, int m, const HadMasks& hm) {
  const int groups = d / m;
  for (int g = threadIdx.x; g < groups; g += blockDim.x) {
    float in[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) in[c] = c < m ? buf[pidx(g * m + c)] : 0.0f;
#pragma unroll
    for (int b = 0; b < 32; ++b) {
      if (b < m) {
        const uint32_t neg = hm.neg[b];
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < 32; ++c) acc += ((neg >> c) & 1u) ? -in[c] : in[c];
        buf[pidx(g * m + b)] = acc;  // in[] holds the group's inputs
      }
    }
  }
}

// One radix-2^R pass of the FWHT over the power-of-two index a (stride m)
// covering index bits [s, s + R).
template <int R>
__device__ __forceinline__ void fwht_pass(float* buf, int n, int m, int s) {
  const int tasks = (m << n) >> R;
  for (int t = threadIdx.x; t < tasks; t += blockDim.x) {
    const int b = t % m;
    const int rest = t / m;
    const int lo = rest & ((1 << s) - 1);
    const int hi = rest >> s;
    const int a0 = lo | (hi << (s + R));
    float v[1 << R];
#pragma unroll
    for (int j = 0; j < (1 << R); ++j) v[j] = buf[pidx((a0 + (j << s)) * m + b)];
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
    for (int j = 0; j < (1 << R); ++j) buf[pidx((a0 + (j << s)) * m + b)] = v[j];
  }
}

// SWIGLU: x is the gate projection and up the up projection; the row is
// SiLU(x) * up in fp32.  m = 1 with a null mask set skips the H_m step.
template <bool SWIGLU>
__global__ __launch_bounds__(kLdsBlock) void had_quant_lds(
    const __half* __restrict__ x, int64_t ld_x, const __half* __restrict__ up, int64_t ld_up,
    int64_t rows, int d, int n, int m, HadMasks hm, const int8_t* __restrict__ signs,
    float clip_ratio, uint8_t* __restrict__ q_out, int64_t ld_q, __half* __restrict__ scale_out,
    float* __restrict__ x_rot, float norm) {
  extern __shared__ float buf[];
  __shared__ float red[kLdsBlock / 64];
  const int chunks = d / 8;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const __half* src = x + row * ld_x;
    // 1. load (and form the gated product), flip signs, widen to fp32
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
      float f[8];
      unpack_half8(*reinterpret_cast<const uint4*>(src + 8 * c), f);
      if (SWIGLU) {
        float u[8];
        unpack_half8(*reinterpret_cast<const uint4*>(up + row * ld_up + 8 * c), u);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = silu_f32(f[i]) * u[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float sgn = (signs && signs[8 * c + i] < 0) ? -1.0f : 1.0f;
        buf[pidx(8 * c + i)] = f[i] * sgn;
      }
    }
    __syncthreads();
    // 2. H_m on each contiguous group of m
    if (m > 1) {
      apply_hm(buf, d, m, hm);
      __syncthreads();
    }
    // 3. FWHT over the 2^n index, radix-32 passes (last pass may be smaller)
    int s = 0;
    while (s < n) {
      const int r = (n - s >= kRadixBits) ? kRadixBits : (n - s);
      switch (r) {
        case 5: fwht_pass<5>(buf, n, m, s); break;
        case 4: fwht_pass<4>(buf, n, m, s); break;
        case 3: fwht_pass<3>(buf, n, m, s); break;
        case 2: fwht_pass<2>(buf, n, m, s); break;
        default: fwht_pass<1>(buf, n, m, s); break;
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

// Raise the dynamic LDS limit of the Kronecker kernel instantiation once.
template <int M, bool CLAMP, bool SWIGLU, int NP>
bool kron_attr_ok() {
  static const bool ok =
      hipFuncSetAttribute(reinterpret_cast<const void*>(had_quant_kron<M, CLAMP, SWIGLU, NP>),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          KronCfg<M, SWIGLU, NP>::LDS_BYTES) == hipSuccess;
  return ok;
}

// The same for the register-butterfly kernel.
template <int M, bool CLAMP, int NP, bool SWIGLU>
bool kront_attr_ok() {
  static const bool ok =
      hipFuncSetAttribute(reinterpret_cast<const void*>(had_quant_kront<M, CLAMP, NP, SWIGLU>),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          KronTCfg<M, NP>::LDS_BYTES) == hipSuccess;
  return ok;
}

// Masks of H_2 (x) H_m (rows and columns i = i0 m + ib, entry
// (-1)^(i0 j0) H_m[ib][jb]) from those of H_m: the Sylvester H_{2^n} is
// H_{2^(n-1)} (x) H_2, so H_{2^n} (x) H_m = H_{2^(n-1)} (x) (H_2 (x) H_m).
HadMasks kron2_masks(const HadMasks& h, int m) {
  HadMasks o{};
  for (int r = 0; r < 2 * m; ++r) {
    const int rb = r % m;
    const uint32_t nz = h.nz[rb], neg = h.neg[rb];
    o.nz[r] = nz | (nz << m);
    o.neg[r] = neg | ((r >= m ? neg ^ nz : neg) << m);
  }
  return o;
}

template <int M, bool CLAMP, bool SWIGLU, int NP>
int launch_kron(const RowSource& src, int64_t rows, const HadMasks& hm, const int8_t* signs,
                float clip_ratio, uint8_t* q_out, int64_t ld_q, __half* scale_out,
                float* x_rot_out, int cus, hipStream_t stream) {
  using C = KronCfg<M, SWIGLU, NP>;
  if (!kron_attr_ok<M, CLAMP, SWIGLU, NP>()) {
    set_error("could not raise the dynamic LDS limit for d = %d", C::D);
    return QUAROT_ERR_HIP;
  }
  // two waves per SIMD (up to 256 VGPRs): one or two blocks per CU
  const int64_t cap = int64_t(cus) * C::BLOCKS_PER_CU;
  const int64_t blocks = rows < cap ? rows : cap;
  const float norm = 1.0f / sqrtf(float(C::D));
  hipLaunchKernelGGL((had_quant_kron<M, CLAMP, SWIGLU, NP>), dim3(unsigned(blocks)),
                     dim3(unsigned(C::THREADS)), C::LDS_BYTES, stream, src.x, src.ld_x, src.up,
                     src.ld_up, rows, signs, hm, clip_ratio, q_out, ld_q, scale_out, x_rot_out,
                     norm);
  return check_launch("had_quant_kron");
}

template <int M, bool CLAMP, int NP, bool SWIGLU>
int launch_kront(const RowSource& src, int64_t rows, const HadMasks& hm, const int8_t* signs,
                 float clip_ratio, uint8_t* q_out, int64_t ld_q, __half* scale_out,
                 float* x_rot_out, int cus, hipStream_t stream) {
  using C = KronTCfg<M, NP>;
  if (!kront_attr_ok<M, CLAMP, NP, SWIGLU>()) {
    set_error("could not raise the dynamic LDS limit for d = %d", C::D);
    return QUAROT_ERR_HIP;
  }
  // two waves per SIMD (up to 256 VGPRs): one or two blocks per CU
  const int64_t cap = int64_t(cus) * C::BLOCKS_PER_CU;
  const int64_t blocks = rows < cap ? rows : cap;
  const float norm = 1.0f / sqrtf(float(C::D));
  hipLaunchKernelGGL((had_quant_kront<M, CLAMP, NP, SWIGLU>), dim3(unsigned(blocks)),
                     dim3(unsigned(C::THREADS)), C::LDS_BYTES, stream, src.x, src.ld_x, src.up,
                     src.ld_up, rows, signs, hm, clip_ratio, q_out, ld_q, scale_out, x_rot_out,
                     norm);
  return check_launch("had_quant_kront");
}

template <int M, bool SWIGLU, int NP = 1024>
int launch_kron_clip(const RowSource& src, int64_t rows, const HadMasks& hm,
                     const int8_t* signs, float clip_ratio, uint8_t* q_out, int64_t ld_q,
                     __half* scale_out, float* x_rot_out, int cus, hipStream_t stream) {
  if (clip_ratio != 1.0f)
    return launch_kron<M, true, SWIGLU, NP>(src, rows, hm, signs, clip_ratio, q_out, ld_q,
                                            scale_out, x_rot_out, cus, stream);
  return launch_kron<M, false, SWIGLU, NP>(src, rows, hm, signs, clip_ratio, q_out, ld_q,
                                           scale_out, x_rot_out, cus, stream);
}

// Rows of 512 groups (plain or gated): the register-butterfly kernel; the
// 1024-group rows: had_quant_kron.
template <int M, bool SWIGLU, int NP = 1024>
int launch_kron_any(const RowSource& src, int64_t rows, const HadMasks& hm,
                    const int8_t* signs, float clip_ratio, uint8_t* q_out, int64_t ld_q,
                    __half* scale_out, float* x_rot_out, int cus, hipStream_t stream) {
  if constexpr (NP != 512) {
    return launch_kron_clip<M, SWIGLU, NP>(src, rows, hm, signs, clip_ratio, q_out, ld_q,
                                           scale_out, x_rot_out, cus, stream);
  } else {
    if (clip_ratio != 1.0f)
      return launch_kront<M, true, NP, SWIGLU>(src, rows, hm, signs, clip_ratio, q_out, ld_q,
                                               scale_out, x_rot_out, cus, stream);
    return launch_kront<M, false, NP, SWIGLU>(src, rows, hm, signs, clip_ratio, q_out, ld_q,
                                              scale_out, x_rot_out, cus, stream);
  }
}

}  // namespace

int launch_had_quant(const RowSource& src, int64_t rows, int d, int n, int m,
                     const HadMasks& hm, const int8_t* signs, float clip_ratio, uint8_t* q_out,
                     int64_t ld_q, __half* scale_out, float* x_rot_out, hipStream_t stream) {
  const int cus = sm_count_cached();
  const bool clamp = clip_ratio != 1.0f;
  const bool gated = src.up != nullptr;
  if (!gated && m == 1 && d <= 256) {
    const int64_t rpb = kQuadBlock / 4;
    int64_t blocks = (rows + rpb - 1) / rpb;
    // at most 2^16 blocks (beyond, blocks loop), far below the 2^32
    // work-item limit of a grid dimension
    const int64_t cap = int64_t(1) << 16;
    if (blocks > cap) blocks = cap;
    const dim3 grid{unsigned(blocks)}, block{unsigned(kQuadBlock)};
#define QR_QUAD(DD, CL)                                                                      \
  hipLaunchKernelGGL((had_quant_quad<DD, CL>), grid, block, 0, stream, src.x, rows, src.ld_x, \
                     signs, clip_ratio, q_out, ld_q, scale_out, x_rot_out)
#define QR_QUAD_D(DD)          \
  if (clamp) QR_QUAD(DD, true); \
  else QR_QUAD(DD, false)
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
  if (!gated && m == 1 && d == 4096) {
    const int64_t cap = int64_t(cus) * 8;  // 16 KiB LDS, two waves per block
    const int64_t blocks = rows < cap ? rows : cap;
    const dim3 grid{unsigned(blocks)}, block{unsigned(kSplitBlock)};
    if (clamp)
      hipLaunchKernelGGL((had_quant_4096_split<true>), grid, block, 0, stream, src.x, rows,
                         src.ld_x, signs, clip_ratio, q_out, ld_q, scale_out, x_rot_out);
    else
      hipLaunchKernelGGL((had_quant_4096_split<false>), grid, block, 0, stream, src.x, rows,
                         src.ld_x, signs, clip_ratio, q_out, ld_q, scale_out, x_rot_out);
    return check_launch("had_quant_4096_split");
  }
  if (m == 12 && d == 1024 * 12) {
    // 512 groups of 24 under H_2 (x) H_12
    const HadMasks h24 = kron2_masks(hm, 12);
    return gated ? launch_kron_any<24, true, 512>(src, rows, h24, signs, clip_ratio, q_out,
                                                  ld_q, scale_out, x_rot_out, cus, stream)
                 : launch_kron_any<24, false, 512>(src, rows, h24, signs, clip_ratio, q_out,
                                                   ld_q, scale_out, x_rot_out, cus, stream);
  }
  if (m == 28 && d == 1024 * 28) {
    return gated ? launch_kron_any<28, true>(src, rows, hm, signs, clip_ratio, q_out, ld_q,
                                             scale_out, x_rot_out, cus, stream)
                 : launch_kron_any<28, false>(src, rows, hm, signs, clip_ratio, q_out, ld_q,
                                              scale_out, x_rot_out, cus, stream);
  }
  const size_t lds = size_t(d + d / 32) * sizeof(float);
  // the generic kernel stages up to 32768 + 1024 floats (132 KiB) in LDS
  static const bool lds_attr_ok = [] {
    const int bytes = (32768 + 1024) * int(sizeof(float));
    bool ok = hipFuncSetAttribute(reinterpret_cast<const void*>(had_quant_lds<false>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                  bytes) == hipSuccess;
    ok &= hipFuncSetAttribute(reinterpret_cast<const void*>(had_quant_lds<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess;
    return ok;
  }();
  if (!lds_attr_ok && lds > 65536) {
    set_error("could not raise the dynamic LDS limit for d = %d", d);
    return QUAROT_ERR_HIP;
  }
  const int64_t per_cu = (lds <= 40 * 1024) ? 4 : (lds <= 76 * 1024 ? 2 : 1);
  const int64_t blocks = rows < int64_t(cus) * per_cu ? rows : int64_t(cus) * per_cu;
  const dim3 grid{unsigned(blocks)}, block{unsigned(kLdsBlock)};
  const float norm = 1.0f / sqrtf(float(d));
  if (gated)
    hipLaunchKernelGGL((had_quant_lds<true>), grid, block, lds, stream, src.x, src.ld_x, src.up,
                       src.ld_up, rows, d, n, m, hm, signs, clip_ratio, q_out, ld_q, scale_out,
                       x_rot_out, norm);
  else
    hipLaunchKernelGGL((had_quant_lds<false>), grid, block, lds, stream, src.x, src.ld_x, src.up,
                       src.ld_up, rows, d, n, m, hm, signs, clip_ratio, q_out, ld_q, scale_out,
                       x_rot_out, norm);
  return check_launch("had_quant_lds");
}

}  // namespace quarot
