// quarot_kv_had_quant: head-wise Hadamard + INT4 quantisation of K and V,
// written into a contiguous quantised cache.
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary), section 3.4 Stage 1d (online head-wise Hadamard I (x) H_{d_h} on
// keys after RoPE; post-RoPE caching), Stage 1c (values rotated head-wise),
// Stage 2c (one quantisation group of 128 per head vector) and the "Append"
// routine of "Kernel Implementation and Hardware Efficiency".
//
// Each (b, h, s) group of D values is one quad_rows row: four lanes, 16-byte
// loads, butterflies in registers and through DPP, codes packed per 8.
#include "quad_rows.h"

namespace quarot {

namespace {

constexpr int kBlock = 256;  // 64 groups per block iteration

struct KvLaunch {
  KvTensorArgs t[2];
  int64_t B, H, S;
  int64_t stride_b, stride_h, stride_s;
  const int8_t* signs;
  int64_t signs_stride_h;
  float clip_ratio;
  int64_t S_cache, pos0;
};

template <int D, bool CLAMP>
__global__ __launch_bounds__(kBlock) void kv_had_quant_kernel(KvLaunch p) {
  constexpr int NC = D / 32;
  const KvTensorArgs t = blockIdx.y ? p.t[1] : p.t[0];
  const int lane_q = threadIdx.x & 3;
  const int64_t groups = p.B * p.H * p.S;
  const int64_t per_block = kBlock / 4;
  uint32_t mask[NC][4];
  int64_t mask_head = -1;
  for (int64_t base = int64_t(blockIdx.x) * per_block; base < groups;
       base += int64_t(gridDim.x) * per_block) {
    const int64_t g = base + (threadIdx.x >> 2);
    const bool active = g < groups;
    const int64_t gg = active ? g : 0;
    const int64_t s = gg % p.S;
    const int64_t bh = gg / p.S;
    const int64_t h = bh % p.H;
    const int64_t b = bh / p.H;
    // signs: one vector per head (stride 0: shared by all heads)
    const int64_t head_key = p.signs_stride_h ? h : 0;
    if (head_key != mask_head) {
      load_sign_masks<NC>(p.signs ? p.signs + head_key * p.signs_stride_h : nullptr, lane_q, mask);
      mask_head = head_key;
    }
    const __half* src = t.src + b * p.stride_b + h * p.stride_h + s * p.stride_s;
    const int64_t slot = bh * p.S_cache + p.pos0 + s;
    quad_row<D, CLAMP>(src, t.q + slot * (D / 2), t.scale + slot, nullptr, mask, lane_q,
                p.clip_ratio, active);
  }
}

}  // namespace

int launch_kv_had_quant(const KvTensorArgs* t, int n_tensors, int64_t B, int64_t H,
                        int64_t S, int D, int64_t stride_b, int64_t stride_h,
                        int64_t stride_s, const int8_t* signs, int64_t signs_stride_h,
                        float clip_ratio, int64_t S_cache, int64_t pos0,
                        hipStream_t stream) {
  KvLaunch p{};
  for (int i = 0; i < n_tensors; ++i) p.t[i] = t[i];
  p.B = B;
  p.H = H;
  p.S = S;
  p.stride_b = stride_b;
  p.stride_h = stride_h;
  p.stride_s = stride_s;
  p.signs = signs;
  p.signs_stride_h = signs_stride_h;
  p.clip_ratio = clip_ratio;
  p.S_cache = S_cache;
  p.pos0 = pos0;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t groups = B * H * S;
  const int64_t per_block = kBlock / 4;
  int64_t blocks = (groups + per_block - 1) / per_block;
  const int64_t cap = int64_t(cus > 0 ? cus : 256) * 8 / n_tensors;
  if (blocks > cap) blocks = cap;
  const dim3 grid{unsigned(blocks), unsigned(n_tensors)}, block{unsigned(kBlock)};
#define QR_KV(DD, CL) hipLaunchKernelGGL((kv_had_quant_kernel<DD, CL>), grid, block, 0, stream, p)
  const bool clamp = clip_ratio != 1.0f;
  switch (D) {
    case 32: if (clamp) QR_KV(32, true); else QR_KV(32, false); break;
    case 64: if (clamp) QR_KV(64, true); else QR_KV(64, false); break;
    case 128: if (clamp) QR_KV(128, true); else QR_KV(128, false); break;
    default: if (clamp) QR_KV(256, true); else QR_KV(256, false); break;
  }
#undef QR_KV
  return check_launch("kv_had_quant");
}

}  // namespace quarot
