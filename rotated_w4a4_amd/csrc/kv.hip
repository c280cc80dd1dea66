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

// n / d for 0 <= n < 2^31 by a multiply-high and a shift (round-up method
// of Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", 1994): with l = ceil(log2 d) and
// mul = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, mul) + n) >> l.
struct FastDiv {
  uint32_t d, mul, shift;
};

FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t mul = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  return FastDiv{d, uint32_t(mul), l};
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& f) {
  return uint32_t((uint64_t(__umulhi(n, f.mul)) + n) >> f.shift);
}

struct KvLaunch {
  KvTensorArgs t[2];
  uint32_t groups;
  FastDiv S, H;
  int64_t stride_b, stride_h, stride_s;
  const int8_t* signs;
  int64_t signs_stride_h;
  float clip_ratio;
  int64_t S_cache, pos0;
};

// Group g = (b H + h) S + s: its fp16 source and its cache slot.
__device__ __forceinline__ void kv_group(const KvLaunch& p, uint32_t g, uint32_t& h,
                                         int64_t& src_off, int64_t& slot) {
  const uint32_t bh = fast_div(g, p.S);
  const uint32_t s = g - bh * p.S.d;
  const uint32_t b = fast_div(bh, p.H);
  h = bh - b * p.H.d;
  src_off = int64_t(b) * p.stride_b + int64_t(h) * p.stride_h + int64_t(s) * p.stride_s;
  slot = int64_t(bh) * p.S_cache + p.pos0 + s;
}

// MODE 0: symmetric (CLAMP when clip < 1); MODE 1: asymmetric with a zero
// point (clipping is part of its range).
template <int D, bool CLAMP, int MODE>
__global__ __launch_bounds__(kBlock) void kv_had_quant_kernel(KvLaunch p) {
  constexpr int NC = D / 32;
  const KvTensorArgs t = blockIdx.y ? p.t[1] : p.t[0];
  const int lane_q = threadIdx.x & 3;
  const uint32_t per_block = kBlock / 4;
  const uint32_t step = gridDim.x * per_block;
  uint4 mask[NC];
  int64_t mask_head = -1;
  uint32_t g = blockIdx.x * per_block + (threadIdx.x >> 2);
  // The grid normally covers every group once (a streaming kernel wants
  // all loads in flight at once rather than a prefetch chain), the loop only
  // serves grids capped below that.
  for (uint32_t base = blockIdx.x * per_block; base < p.groups; base += step, g += step) {
    const bool active = g < p.groups;
    uint32_t h;
    int64_t src_off, slot;
    kv_group(p, active ? g : 0, h, src_off, slot);
    uint4 raw[NC];
    quad_load<D>(t.src + src_off, lane_q, raw);
    // signs: one vector per head (stride 0: shared by all heads)
    const int64_t head_key = p.signs_stride_h ? int64_t(h) : 0;
    if (head_key != mask_head) {
      load_sign_masks<NC>(p.signs ? p.signs + head_key * p.signs_stride_h : nullptr, lane_q, mask);
      mask_head = head_key;
    }
    // optional rotated copy, dense [B, H, S, D]: group g's row
    float* rot = t.rot ? t.rot + int64_t(active ? g : 0) * D : nullptr;
    if (MODE == 0)
      quad_row<D, CLAMP>(raw, t.q + slot * (D / 2), t.scale + slot, rot, mask, lane_q,
                         p.clip_ratio, active);
    else
      quad_row_asym<D>(raw, t.q + slot * (D / 2), t.scale + slot, t.zero + slot, rot, mask,
                       lane_q, p.clip_ratio, active);
  }
}

}  // namespace

int launch_kv_had_quant(const KvTensorArgs* t, int n_tensors, int64_t B, int64_t H,
                        int64_t S, int D, int64_t stride_b, int64_t stride_h,
                        int64_t stride_s, const int8_t* signs, int64_t signs_stride_h,
                        int mode, float clip_ratio, int64_t S_cache, int64_t pos0,
                        hipStream_t stream) {
  KvLaunch p{};
  for (int i = 0; i < n_tensors; ++i) p.t[i] = t[i];
  p.groups = uint32_t(B * H * S);  // < 2^31, checked by the caller
  p.S = make_fastdiv(uint32_t(S));
  p.H = make_fastdiv(uint32_t(H));
  p.stride_b = stride_b;
  p.stride_h = stride_h;
  p.stride_s = stride_s;
  p.signs = signs;
  p.signs_stride_h = signs_stride_h;
  p.clip_ratio = clip_ratio;
  p.S_cache = S_cache;
  p.pos0 = pos0;
  const int64_t groups = B * H * S;
  const int64_t per_block = kBlock / 4;
  int64_t blocks = (groups + per_block - 1) / per_block;
  // at most 2^16 blocks (beyond, blocks loop), far below the 2^32 work-item
  // limit of a grid dimension
  const int64_t cap = int64_t(1) << 16;
  if (blocks > cap) blocks = cap;
  const dim3 grid{unsigned(blocks), unsigned(n_tensors)}, block{unsigned(kBlock)};
#define QR_KV(DD, CL, MD) \
  hipLaunchKernelGGL((kv_had_quant_kernel<DD, CL, MD>), grid, block, 0, stream, p)
#define QR_KV_D(DD)                          \
  if (mode == 1) QR_KV(DD, false, 1);        \
  else if (clamp) QR_KV(DD, true, 0);        \
  else QR_KV(DD, false, 0)
  const bool clamp = clip_ratio != 1.0f;
  switch (D) {
    case 32: QR_KV_D(32); break;
    case 64: QR_KV_D(64); break;
    case 128: QR_KV_D(128); break;
    default: QR_KV_D(256); break;
  }
#undef QR_KV_D
#undef QR_KV
  return check_launch("kv_had_quant");
}

}  // namespace quarot
