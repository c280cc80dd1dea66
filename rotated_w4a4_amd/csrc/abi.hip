// C ABI of libquarot: argument validation, status strings, and dispatch to
// the kernel launchers.  Every check here runs on the host before any HIP
// call, so a rejected call never touches the device or the stream.
#include <cstring>

#include "common.h"
#include "cross_head.h"
#include "decode.h"

namespace quarot {

namespace {
thread_local char g_last_error[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

void clear_error() { g_last_error[0] = '\0'; }

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return QUAROT_ERR_HIP;
  }
  return QUAROT_OK;
}

namespace {

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int log2_exact(int64_t v) {
  int n = 0;
  while ((int64_t(1) << n) < v) ++n;
  return n;
}

bool clip_ok(float c) { return c > 0.0f && c <= 1.0f; }  // also rejects NaN

}  // namespace
}  // namespace quarot

using namespace quarot;

extern "C" {

const char* quarot_status_string(int status) {
  switch (status) {
    case QUAROT_OK: return "ok";
    case QUAROT_ERR_INVALID: return "invalid argument";
    case QUAROT_ERR_UNSUPPORTED: return "unsupported shape or mode";
    case QUAROT_ERR_MISALIGNED: return "misaligned pointer or stride";
    case QUAROT_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* quarot_last_error(void) { return g_last_error; }

int quarot_hadamard_factor(int32_t m, int8_t* out_host) {
  clear_error();
  QR_CHECK_ARG(out_host != nullptr, QUAROT_ERR_INVALID, "out_host is NULL");
  switch (m) {
    case 1: out_host[0] = 1; return QUAROT_OK;
    case 12: std::memcpy(out_host, HadTable<12>::value.v, 12 * 12); return QUAROT_OK;
    case 28: std::memcpy(out_host, HadTable<28>::value.v, 28 * 28); return QUAROT_OK;
    default:
      set_error("no built-in Hadamard factor of order %d (have 1, 12, 28)", m);
      return QUAROT_ERR_UNSUPPORTED;
  }
}

namespace {

// The caller's small Hadamard factor (host memory), validated and turned
// into the kernels' bit masks: NULL iff m == 1; m a multiple of 4 up to 32;
// entries +1/-1 with H H^T = m I in exact integer arithmetic.
int had_masks_checked(int32_t m, const int8_t* had_m, HadMasks* out) {
  *out = HadMasks{};
  if (m == 1) {
    QR_CHECK_ARG(had_m == nullptr, QUAROT_ERR_INVALID, "had_m must be NULL when m = 1");
    out->nz[0] = 1u;
    return QUAROT_OK;
  }
  QR_CHECK_ARG(m >= 4 && m <= 32 && m % 4 == 0, QUAROT_ERR_UNSUPPORTED,
               "m = %d: the small Hadamard factor must have order 1 or a multiple of 4 up to 32",
               m);
  QR_CHECK_ARG(had_m != nullptr, QUAROT_ERR_INVALID, "had_m is required for m = %d", m);
  for (int i = 0; i < m; ++i)
    for (int j = 0; j < m; ++j) {
      const int e = had_m[i * m + j];
      QR_CHECK_ARG(e == 1 || e == -1, QUAROT_ERR_INVALID,
                   "had_m[%d][%d] = %d: entries must be +1 or -1", i, j, e);
    }
  for (int i = 0; i < m; ++i)
    for (int j = i; j < m; ++j) {
      int dot = 0;
      for (int k = 0; k < m; ++k) dot += had_m[i * m + k] * had_m[j * m + k];
      QR_CHECK_ARG(dot == (i == j ? m : 0), QUAROT_ERR_INVALID,
                   "had_m is not a Hadamard matrix: rows %d and %d have dot product %d", i, j,
                   dot);
    }
  for (int i = 0; i < m; ++i)
    for (int j = 0; j < m; ++j) {
      out->nz[i] |= 1u << j;
      if (had_m[i * m + j] < 0) out->neg[i] |= 1u << j;
    }
  return QUAROT_OK;
}

// Shared checks and dispatch of the rotate+quant entry points.  up != NULL:
// the rows are SiLU(x) * up.
int had_quant_checked(const void* x, int64_t ld_x, const void* up, int64_t ld_up, int64_t rows,
                      int64_t d, const int8_t* signs, int32_t m, const int8_t* had_m,
                      float clip_ratio, uint8_t* q_out, int64_t ld_q, void* scale_out,
                      float* x_rot_out, void* stream) {
  QR_CHECK_ARG(rows >= 0, QUAROT_ERR_INVALID, "rows = %lld < 0", (long long)rows);
  QR_CHECK_ARG(d > 0, QUAROT_ERR_INVALID, "d = %lld <= 0", (long long)d);
  QR_CHECK_ARG(clip_ok(clip_ratio), QUAROT_ERR_INVALID, "clip_ratio must be in (0, 1]");
  HadMasks hm;
  const int st = had_masks_checked(m, had_m, &hm);
  if (st != QUAROT_OK) return st;
  QR_CHECK_ARG(d % m == 0 && is_pow2(d / m), QUAROT_ERR_UNSUPPORTED,
               "d = %lld is not 2^n * %d", (long long)d, m);
  QR_CHECK_ARG(d % 32 == 0 && d <= 32768, QUAROT_ERR_UNSUPPORTED,
               "d = %lld: need d %% 32 == 0 and d <= 32768", (long long)d);
  QR_CHECK_ARG(ld_x >= d, QUAROT_ERR_INVALID, "row stride %lld < d", (long long)ld_x);
  QR_CHECK_ARG(up == nullptr || ld_up >= d, QUAROT_ERR_INVALID, "ld_up = %lld < d",
               (long long)ld_up);
  QR_CHECK_ARG(ld_q >= d / 2, QUAROT_ERR_INVALID, "ld_q = %lld < d/2", (long long)ld_q);
  if (rows == 0) return QUAROT_OK;
  QR_CHECK_ARG(x && q_out && scale_out, QUAROT_ERR_INVALID,
               "the input, q_out and scale_out are required");
  QR_CHECK_ARG(aligned(x, 16) && ld_x % 8 == 0, QUAROT_ERR_MISALIGNED,
               "the input must be 16-byte aligned with a row stride %% 8 == 0");
  QR_CHECK_ARG(up == nullptr || (aligned(up, 16) && ld_up % 8 == 0), QUAROT_ERR_MISALIGNED,
               "up must be 16-byte aligned with ld_up %% 8 == 0");
  QR_CHECK_ARG(aligned(q_out, 16) && ld_q % 16 == 0, QUAROT_ERR_MISALIGNED,
               "q_out must be 16-byte aligned with ld_q %% 16 == 0");
  QR_CHECK_ARG(aligned(scale_out, 2), QUAROT_ERR_MISALIGNED, "scale_out must be 2-byte aligned");
  QR_CHECK_ARG(x_rot_out == nullptr || aligned(x_rot_out, 16), QUAROT_ERR_MISALIGNED,
               "x_rot_out must be 16-byte aligned");
  QR_CHECK_ARG(rows <= (int64_t(1) << 31) - 1, QUAROT_ERR_UNSUPPORTED, "rows too large");
  const int n = log2_exact(d / m);
  const RowSource src{static_cast<const __half*>(x), ld_x, static_cast<const __half*>(up),
                      ld_up};
  return launch_had_quant(src, rows, int(d), n, m, hm, signs, clip_ratio, q_out, ld_q,
                          static_cast<__half*>(scale_out), x_rot_out,
                          static_cast<hipStream_t>(stream));
}

}  // namespace

int quarot_had_quant(const void* x, int64_t rows, int64_t d, int64_t ld_x,
                     const int8_t* signs, int32_t m, const int8_t* had_m, float clip_ratio,
                     uint8_t* q_out, int64_t ld_q, void* scale_out,
                     float* x_rot_out, void* stream) {
  clear_error();
  return had_quant_checked(x, ld_x, nullptr, 0, rows, d, signs, m, had_m, clip_ratio, q_out,
                           ld_q, scale_out, x_rot_out, stream);
}

int quarot_swiglu_had_quant(const void* gate, const void* up, int64_t rows, int64_t d,
                            int64_t ld_gate, int64_t ld_up, const int8_t* signs, int32_t m,
                            const int8_t* had_m, float clip_ratio, uint8_t* q_out, int64_t ld_q,
                            void* scale_out, float* x_rot_out, void* stream) {
  clear_error();
  QR_CHECK_ARG(rows == 0 || up != nullptr, QUAROT_ERR_INVALID, "up is required");
  return had_quant_checked(gate, ld_gate, up, ld_up, rows, d, signs, m, had_m, clip_ratio, q_out,
                           ld_q, scale_out, x_rot_out, stream);
}

int quarot_cross_head_had_quant(const void* z, int64_t rows, int64_t n_heads, int64_t head_dim,
                                int64_t ld_z, float clip_ratio, uint8_t* q_out, int64_t ld_q,
                                void* scale_out, float* z_rot_out, void* stream) {
  clear_error();
  QR_CHECK_ARG(rows >= 0, QUAROT_ERR_INVALID, "rows = %lld < 0", (long long)rows);
  QR_CHECK_ARG(n_heads > 0 && head_dim > 0, QUAROT_ERR_INVALID, "n_heads and head_dim must be > 0");
  QR_CHECK_ARG(clip_ok(clip_ratio), QUAROT_ERR_INVALID, "clip_ratio must be in (0, 1]");
  QR_CHECK_ARG(head_dim == 128, QUAROT_ERR_UNSUPPORTED, "head_dim = %lld: supported is 128",
               (long long)head_dim);
  QR_CHECK_ARG(is_pow2(n_heads) && n_heads <= 64, QUAROT_ERR_UNSUPPORTED,
               "n_heads = %lld: need a power of two <= 64", (long long)n_heads);
  const int64_t d = n_heads * head_dim;
  QR_CHECK_ARG(ld_z >= d, QUAROT_ERR_INVALID, "ld_z = %lld < n_heads * head_dim", (long long)ld_z);
  QR_CHECK_ARG(ld_q >= d / 2, QUAROT_ERR_INVALID, "ld_q = %lld < n_heads * head_dim / 2",
               (long long)ld_q);
  if (rows == 0) return QUAROT_OK;
  QR_CHECK_ARG(z && q_out && scale_out, QUAROT_ERR_INVALID, "z, q_out and scale_out are required");
  QR_CHECK_ARG(aligned(z, 4) && ld_z % 2 == 0, QUAROT_ERR_MISALIGNED,
               "z must be 4-byte aligned with an even ld_z");
  QR_CHECK_ARG(aligned(scale_out, 2), QUAROT_ERR_MISALIGNED, "scale_out must be 2-byte aligned");
  QR_CHECK_ARG(z_rot_out == nullptr || aligned(z_rot_out, 8), QUAROT_ERR_MISALIGNED,
               "z_rot_out must be 8-byte aligned");
  QR_CHECK_ARG(rows <= (int64_t(1) << 31) - 1, QUAROT_ERR_UNSUPPORTED, "rows too large");
  return launch_cross_head_quant(static_cast<const __half*>(z), rows, int(n_heads), ld_z,
                                 clip_ratio, q_out, ld_q, static_cast<__half*>(scale_out),
                                 z_rot_out, static_cast<hipStream_t>(stream));
}

int quarot_w4a4_gemm(const uint8_t* a_q, int64_t lda, const void* a_scale,
                     const uint8_t* b_q, int64_t ldb, const void* b_scale,
                     int64_t M, int64_t N, int64_t K,
                     void* c, int64_t ldc, int32_t* acc_out, int64_t ld_acc,
                     void* stream) {
  clear_error();
  QR_CHECK_ARG(M >= 0 && N >= 0, QUAROT_ERR_INVALID, "M, N must be >= 0");
  QR_CHECK_ARG(K > 0, QUAROT_ERR_INVALID, "K must be > 0");
  QR_CHECK_ARG(K % 32 == 0, QUAROT_ERR_UNSUPPORTED, "K = %lld: need K %% 32 == 0", (long long)K);
  QR_CHECK_ARG(K <= 65536, QUAROT_ERR_UNSUPPORTED, "K = %lld > 65536", (long long)K);
  QR_CHECK_ARG(lda >= K / 2 && ldb >= K / 2, QUAROT_ERR_INVALID, "lda, ldb must be >= K/2");
  QR_CHECK_ARG(ldc >= N, QUAROT_ERR_INVALID, "ldc must be >= N");
  QR_CHECK_ARG(acc_out == nullptr || ld_acc >= N, QUAROT_ERR_INVALID, "ld_acc must be >= N");
  if (M == 0 || N == 0) return QUAROT_OK;
  QR_CHECK_ARG(a_q && a_scale && b_q && b_scale && c, QUAROT_ERR_INVALID,
               "a_q, a_scale, b_q, b_scale and c are required");
  QR_CHECK_ARG(aligned(a_q, 16) && aligned(b_q, 16) && lda % 16 == 0 && ldb % 16 == 0,
               QUAROT_ERR_MISALIGNED, "a_q/b_q must be 16-byte aligned with lda, ldb %% 16 == 0");
  QR_CHECK_ARG(aligned(a_scale, 2) && aligned(b_scale, 2), QUAROT_ERR_MISALIGNED,
               "scales must be 2-byte aligned");
  QR_CHECK_ARG(aligned(c, 2), QUAROT_ERR_MISALIGNED, "c must be 2-byte aligned");
  QR_CHECK_ARG(acc_out == nullptr || aligned(acc_out, 4), QUAROT_ERR_MISALIGNED,
               "acc_out must be 4-byte aligned");
  QR_CHECK_ARG(M < (int64_t(1) << 31) && N < (int64_t(1) << 31), QUAROT_ERR_UNSUPPORTED,
               "M, N too large");
  return launch_w4a4_gemm(a_q, lda, static_cast<const __half*>(a_scale), b_q, ldb,
                          static_cast<const __half*>(b_scale), M, N, K,
                          static_cast<__half*>(c), ldc, acc_out, ld_acc,
                          static_cast<hipStream_t>(stream));
}

int quarot_kv_had_quant(const void* k, const void* v,
                        int64_t B, int64_t H, int64_t S, int64_t D,
                        int64_t stride_b, int64_t stride_h, int64_t stride_s,
                        const int8_t* signs, int64_t signs_stride_h,
                        int32_t mode, float clip_ratio,
                        uint8_t* k_q, void* k_scale, void* k_zero,
                        uint8_t* v_q, void* v_scale, void* v_zero,
                        int64_t S_cache, int64_t pos0, float* k_rot_out, float* v_rot_out,
                        void* stream) {
  clear_error();
  QR_CHECK_ARG(B >= 0 && H >= 0 && S >= 0, QUAROT_ERR_INVALID, "B, H, S must be >= 0");
  QR_CHECK_ARG(D == 32 || D == 64 || D == 128 || D == 256, QUAROT_ERR_UNSUPPORTED,
               "D = %lld: supported head dims are 32, 64, 128, 256", (long long)D);
  QR_CHECK_ARG(mode == 0 || mode == 1, QUAROT_ERR_INVALID, "mode must be 0 or 1");
  QR_CHECK_ARG(clip_ok(clip_ratio), QUAROT_ERR_INVALID, "clip_ratio must be in (0, 1]");
  QR_CHECK_ARG(stride_b >= 0 && stride_h >= 0 && stride_s >= 0 && signs_stride_h >= 0,
               QUAROT_ERR_INVALID, "strides must be >= 0");
  QR_CHECK_ARG(pos0 >= 0 && S_cache >= 0 && pos0 + S <= S_cache, QUAROT_ERR_INVALID,
               "need 0 <= pos0 and pos0 + S <= S_cache");
  QR_CHECK_ARG(k != nullptr || v != nullptr, QUAROT_ERR_INVALID, "k and v are both NULL");
  if (B == 0 || H == 0 || S == 0) return QUAROT_OK;
  QR_CHECK_ARG(stride_b % 8 == 0 && stride_h % 8 == 0 && stride_s % 8 == 0, QUAROT_ERR_MISALIGNED,
               "strides must be multiples of 8 elements");
  KvTensorArgs t[2];
  int nt = 0;
  const void* srcs[2] = {k, v};
  uint8_t* qs[2] = {k_q, v_q};
  void* ss[2] = {k_scale, v_scale};
  void* zs[2] = {k_zero, v_zero};
  float* rs[2] = {k_rot_out, v_rot_out};
  for (int i = 0; i < 2; ++i) {
    if (!srcs[i]) continue;
    QR_CHECK_ARG(qs[i] && ss[i], QUAROT_ERR_INVALID, "%s_q and %s_scale are required",
                 i ? "v" : "k", i ? "v" : "k");
    QR_CHECK_ARG(mode == 0 || zs[i], QUAROT_ERR_INVALID, "mode 1 needs %s_zero",
                 i ? "v" : "k");
    QR_CHECK_ARG(aligned(srcs[i], 16) && aligned(qs[i], 16) && aligned(ss[i], 2) &&
                     (mode == 0 || aligned(zs[i], 2)),
                 QUAROT_ERR_MISALIGNED, "inputs and code buffers must be 16-byte aligned");
    QR_CHECK_ARG(rs[i] == nullptr || aligned(rs[i], 16), QUAROT_ERR_MISALIGNED,
                 "%s_rot_out must be 16-byte aligned", i ? "v" : "k");
    t[nt++] = KvTensorArgs{static_cast<const __half*>(srcs[i]), qs[i],
                           static_cast<__half*>(ss[i]),
                           mode == 1 ? static_cast<__half*>(zs[i]) : nullptr, rs[i]};
  }
  QR_CHECK_ARG(B * H * S < (int64_t(1) << 31), QUAROT_ERR_UNSUPPORTED, "too many groups");
  return launch_kv_had_quant(t, nt, B, H, S, int(D), stride_b, stride_h, stride_s, signs,
                             signs_stride_h, int(mode), clip_ratio, S_cache, pos0,
                             static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Shared checks of the decode entry point and its workspace query.
int decode_shape_ok(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t max_len) {
  QR_CHECK_ARG(B >= 0, QUAROT_ERR_INVALID, "B = %lld < 0", (long long)B);
  QR_CHECK_ARG(Hq > 0 && Hkv > 0, QUAROT_ERR_INVALID, "Hq and Hkv must be > 0");
  QR_CHECK_ARG(Hq % Hkv == 0, QUAROT_ERR_INVALID, "Hq = %lld is not a multiple of Hkv = %lld",
               (long long)Hq, (long long)Hkv);
  QR_CHECK_ARG(D == 128, QUAROT_ERR_UNSUPPORTED, "D = %lld: the decode kernel needs D = 128",
               (long long)D);
  QR_CHECK_ARG(Hq / Hkv <= 8, QUAROT_ERR_UNSUPPORTED, "Hq / Hkv = %lld > 8",
               (long long)(Hq / Hkv));
  QR_CHECK_ARG(max_len >= 1, QUAROT_ERR_INVALID, "max_len = %lld < 1", (long long)max_len);
  QR_CHECK_ARG(max_len <= (int64_t(1) << 24), QUAROT_ERR_UNSUPPORTED,
               "max_len = %lld > 2^24 (32-bit buffer offsets)", (long long)max_len);
  // one 256-thread workgroup per (b, kv head) in the first grid dimension,
  // whose work-item count must stay below 2^32
  QR_CHECK_ARG(B * Hkv < (int64_t(1) << 24), QUAROT_ERR_UNSUPPORTED, "B * Hkv = %lld >= 2^24",
               (long long)(B * Hkv));
  return QUAROT_OK;
}

}  // namespace

extern "C" {

int64_t quarot_kv_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                         int64_t max_len) {
  clear_error();
  const int st = decode_shape_ok(B, Hq, Hkv, D, max_len);
  if (st != QUAROT_OK) return st;
  return decode_workspace_bytes(B, Hq, Hkv, max_len);
}

namespace {

// Shared validation and launch of both decode entry points.  noalloc: the
// partials go to the library's scratch array instead of the workspace.
int decode_checked(const void* q, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                   const int8_t* signs, int64_t signs_stride_h, int32_t mode,
                   const uint8_t* k_q, const void* k_scale, const void* k_zero,
                   const uint8_t* v_q, const void* v_scale, const void* v_zero,
                   int64_t S_cache, int64_t max_len, const int32_t* lengths, float sm_scale,
                   int32_t cross_head, void* out, float* out_f32, void* workspace,
                   int64_t workspace_bytes, bool noalloc, void* stream) {
  int st = decode_shape_ok(B, Hq, Hkv, D, max_len);
  if (st != QUAROT_OK) return st;
  QR_CHECK_ARG(mode == 0 || mode == 1, QUAROT_ERR_INVALID, "mode must be 0 or 1");
  QR_CHECK_ARG(cross_head == 0 || cross_head == 1, QUAROT_ERR_INVALID, "cross_head must be 0 or 1");
  QR_CHECK_ARG(sm_scale > 0.0f && sm_scale < INFINITY, QUAROT_ERR_INVALID,
               "sm_scale must be finite and > 0");
  QR_CHECK_ARG(signs_stride_h >= 0, QUAROT_ERR_INVALID, "signs_stride_h must be >= 0");
  QR_CHECK_ARG(max_len <= S_cache, QUAROT_ERR_INVALID, "max_len = %lld > S_cache = %lld",
               (long long)max_len, (long long)S_cache);
  QR_CHECK_ARG(cross_head == 0 || (is_pow2(Hq) && Hq <= 256), QUAROT_ERR_UNSUPPORTED,
               "cross_head needs Hq a power of two <= 256 (Hq = %lld)", (long long)Hq);
  const int64_t need = decode_workspace_bytes(B, Hq, Hkv, max_len);
  QR_CHECK_ARG(!noalloc || need <= QUAROT_DECODE_SCRATCH_BYTES, QUAROT_ERR_UNSUPPORTED,
               "these sizes need %lld bytes of partials; the allocation-free entry point holds "
               "%lld (use quarot_kv_decode_attention with a workspace)",
               (long long)need, (long long)QUAROT_DECODE_SCRATCH_BYTES);
  if (B == 0) return QUAROT_OK;
  QR_CHECK_ARG(q && k_q && k_scale && v_q && v_scale && out, QUAROT_ERR_INVALID,
               "q, k_q, k_scale, v_q, v_scale and out are required");
  QR_CHECK_ARG(mode == 0 || (k_zero && v_zero), QUAROT_ERR_INVALID, "mode 1 needs k_zero and v_zero");
  if (!noalloc) {
    QR_CHECK_ARG(workspace && workspace_bytes >= need, QUAROT_ERR_INVALID,
                 "workspace of %lld bytes needed, %lld given", (long long)need,
                 (long long)workspace_bytes);
    QR_CHECK_ARG(aligned(workspace, 16), QUAROT_ERR_MISALIGNED,
                 "workspace must be 16-byte aligned");
  }
  QR_CHECK_ARG(aligned(q, 16) && aligned(k_q, 16) && aligned(v_q, 16),
               QUAROT_ERR_MISALIGNED, "q, k_q and v_q must be 16-byte aligned");
  QR_CHECK_ARG(aligned(k_scale, 2) && aligned(v_scale, 2) && aligned(out, 2) &&
                   (mode == 0 || (aligned(k_zero, 2) && aligned(v_zero, 2))),
               QUAROT_ERR_MISALIGNED, "fp16 buffers must be 2-byte aligned");
  QR_CHECK_ARG(out_f32 == nullptr || aligned(out_f32, 4), QUAROT_ERR_MISALIGNED,
               "out_f32 must be 4-byte aligned");
  QR_CHECK_ARG(lengths == nullptr || aligned(lengths, 4), QUAROT_ERR_MISALIGNED,
               "lengths must be 4-byte aligned");
  if (noalloc) {
    st = decode_scratch(&workspace);
    if (st != QUAROT_OK) return st;
  }
  DecodeTensors t{};
  t.q = static_cast<const __half*>(q);
  t.signs = signs;
  t.signs_stride_h = signs_stride_h;
  t.k_q = k_q;
  t.k_scale = static_cast<const __half*>(k_scale);
  t.k_zero = mode == 1 ? static_cast<const __half*>(k_zero) : nullptr;
  t.v_q = v_q;
  t.v_scale = static_cast<const __half*>(v_scale);
  t.v_zero = mode == 1 ? static_cast<const __half*>(v_zero) : nullptr;
  t.lengths = lengths;
  t.out = static_cast<__half*>(out);
  t.out_f32 = out_f32;
  t.workspace = workspace;
  return launch_kv_decode(t, B, Hq, Hkv, S_cache, max_len, sm_scale, int(mode), cross_head != 0,
                          static_cast<hipStream_t>(stream));
}

}  // namespace

int quarot_kv_decode_attention(const void* q, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                               const int8_t* signs, int64_t signs_stride_h, int32_t mode,
                               const uint8_t* k_q, const void* k_scale, const void* k_zero,
                               const uint8_t* v_q, const void* v_scale, const void* v_zero,
                               int64_t S_cache, int64_t max_len, const int32_t* lengths,
                               float sm_scale, int32_t cross_head,
                               void* out, float* out_f32,
                               void* workspace, int64_t workspace_bytes, void* stream) {
  clear_error();
  return decode_checked(q, B, Hq, Hkv, D, signs, signs_stride_h, mode, k_q, k_scale, k_zero, v_q,
                        v_scale, v_zero, S_cache, max_len, lengths, sm_scale, cross_head, out,
                        out_f32, workspace, workspace_bytes, false, stream);
}

int quarot_kv_decode_attention_noalloc(const void* q, int64_t B, int64_t Hq, int64_t Hkv,
                                       int64_t D, const int8_t* signs, int64_t signs_stride_h,
                                       int32_t mode, const uint8_t* k_q, const void* k_scale,
                                       const void* k_zero, const uint8_t* v_q,
                                       const void* v_scale, const void* v_zero, int64_t S_cache,
                                       int64_t max_len, const int32_t* lengths, float sm_scale,
                                       int32_t cross_head, void* out, float* out_f32,
                                       void* stream) {
  clear_error();
  return decode_checked(q, B, Hq, Hkv, D, signs, signs_stride_h, mode, k_q, k_scale, k_zero, v_q,
                        v_scale, v_zero, S_cache, max_len, lengths, sm_scale, cross_head, out,
                        out_f32, nullptr, 0, true, stream);
}

}  // extern "C"
