// Internal helpers shared by the HIP sources of libquarot (not installed).
//
// Contents: status/last-error plumbing, the compile-time Paley type-I
// Hadamard matrices of order 12 and 28 (handed out by quarot_hadamard_factor),
// the H_m bit masks and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>

#include "quarot.h"

namespace quarot {

// ---------------------------------------------------------------------------
// Error plumbing: a thread-local message plus the status code.
// ---------------------------------------------------------------------------
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

#define QR_CHECK_ARG(cond, status, ...)      \
  do {                                       \
    if (!(cond)) {                           \
      ::quarot::set_error(__VA_ARGS__);      \
      return (status);                       \
    }                                        \
  } while (0)

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Launch-error check after hipLaunchKernelGGL.
int check_launch(const char* what);

// ---------------------------------------------------------------------------
// Paley construction I, evaluated at compile time.
//
// "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
// summary), section 3.4 Stage 1a: for d = 2^n * m the rotation uses
// H_{2^n} (x) H_m with a known Hadamard matrix H_m; the QuaRot paper-viz
// explainer uses a Paley block of size 12.  Paley I gives order q + 1 for a
// prime power q = 3 (mod 4):
//   Q[i][j] = chi(e_i - e_j)  (chi: quadratic character of GF(q))
//   S = [[0, 1^T], [-1, Q]],  H = I + S.
// Field elements are indexed 0..q-1; for q = p^k the element with index i is
// sum_k c_k t^k with c_k the base-p digits of i (least significant first);
// GF(27) = GF(3)[t] / (t^3 + 2t + 2).
// ---------------------------------------------------------------------------
struct GfDesc {
  int p, k, q;
  int mod_low[3];  // t^k = -(mod_low[0] + mod_low[1] t + mod_low[2] t^2)
};

constexpr GfDesc gf_for(int q) {
  if (q == 27) return GfDesc{3, 3, 27, {2, 2, 0}};
  return GfDesc{q, 1, q, {0, 0, 0}};
}

constexpr int gf_sub(const GfDesc& f, int a, int b) {
  int out = 0, scale = 1;
  for (int i = 0; i < f.k; ++i) {
    int da = a % f.p, db = b % f.p;
    a /= f.p;
    b /= f.p;
    out += ((da - db + f.p) % f.p) * scale;
    scale *= f.p;
  }
  return out;
}

constexpr int gf_mul(const GfDesc& f, int a, int b) {
  int da[3] = {0, 0, 0}, db[3] = {0, 0, 0};
  for (int i = 0; i < f.k; ++i) {
    da[i] = a % f.p;
    a /= f.p;
    db[i] = b % f.p;
    b /= f.p;
  }
  int prod[5] = {0, 0, 0, 0, 0};
  for (int i = 0; i < f.k; ++i)
    for (int j = 0; j < f.k; ++j) prod[i + j] = (prod[i + j] + da[i] * db[j]) % f.p;
  for (int deg = 2 * f.k - 2; deg >= f.k; --deg) {
    const int c = prod[deg];
    if (c) {
      prod[deg] = 0;
      for (int j = 0; j < f.k; ++j)
        prod[deg - f.k + j] = ((prod[deg - f.k + j] - c * f.mod_low[j]) % f.p + f.p) % f.p;
    }
  }
  int out = 0, scale = 1;
  for (int i = 0; i < f.k; ++i) {
    out += prod[i] * scale;
    scale *= f.p;
  }
  return out;
}

constexpr int gf_chi(const GfDesc& f, int a) {
  if (a == 0) return 0;
  for (int x = 1; x < f.q; ++x)
    if (gf_mul(f, x, x) == a) return 1;
  return -1;
}

template <int M>
struct HadFactor {
  signed char v[M][M];
};

template <int M>
constexpr HadFactor<M> make_had_factor() {
  HadFactor<M> h{};
  if (M == 1) {
    h.v[0][0] = 1;
    return h;
  }
  const GfDesc f = gf_for(M - 1);
  const int q = M - 1;
  for (int i = 0; i < M; ++i)
    for (int j = 0; j < M; ++j) {
      int s = 0;
      if (i == 0 && j == 0) s = 0;
      else if (i == 0) s = 1;
      else if (j == 0) s = -1;
      else s = gf_chi(f, gf_sub(f, i - 1, j - 1));
      h.v[i][j] = static_cast<signed char>((i == j ? 1 : 0) + s);
    }
  (void)q;
  return h;
}

template <int M>
struct HadTable {
  static constexpr HadFactor<M> value = make_had_factor<M>();
};

// Compile-time sanity: each factor is orthogonal with H H^T = M I.
template <int M>
constexpr bool had_factor_ok() {
  constexpr HadFactor<M> h = make_had_factor<M>();
  for (int i = 0; i < M; ++i)
    for (int j = 0; j < M; ++j) {
      int s = 0;
      for (int k = 0; k < M; ++k) s += h.v[i][k] * h.v[j][k];
      if (s != (i == j ? M : 0)) return false;
    }
  return true;
}
static_assert(had_factor_ok<12>(), "H_12 is not Hadamard");
static_assert(had_factor_ok<28>(), "H_28 is not Hadamard");

// ---------------------------------------------------------------------------
// The small Hadamard factor H_m as bit masks over columns, rows and columns
// padded to 32 with zeros: row r has entry -1 where bit c of neg[r] is set,
// +1 where only bit c of nz[r] is set, 0 where neither is.  Built on the
// host from the caller's matrix and handed to the kernels by value.
// ---------------------------------------------------------------------------
struct HadMasks {
  uint32_t neg[32];
  uint32_t nz[32];
};

// The rows a rotate+quant launch reads: x (fp16, row stride ld_x), or, with
// up != nullptr, the gated product SiLU(x) * up formed on the fly (x is then
// the gate projection, up the up projection, row stride ld_up).
struct RowSource {
  const __half* x;
  int64_t ld_x;
  const __half* up;
  int64_t ld_up;
};

// ---------------------------------------------------------------------------
// Kernel launchers (one per .hip file); arguments already validated.
// ---------------------------------------------------------------------------
int launch_had_quant(const RowSource& src, int64_t rows, int d, int n, int m,
                     const HadMasks& hm, const int8_t* signs, float clip_ratio, uint8_t* q_out,
                     int64_t ld_q, __half* scale_out, float* x_rot_out, hipStream_t stream);

int launch_w4a4_gemm(const uint8_t* a_q, int64_t lda, const __half* a_scale,
                     const uint8_t* b_q, int64_t ldb, const __half* b_scale,
                     int64_t M, int64_t N, int64_t K, __half* c, int64_t ldc,
                     int32_t* acc_out, int64_t ld_acc, hipStream_t stream);

struct KvTensorArgs {
  const __half* src;
  uint8_t* q;
  __half* scale;
  __half* zero;  // asymmetric mode only
  float* rot;    // optional fp32 [B, H, S, D] copy of the rotated groups
};

int launch_kv_had_quant(const KvTensorArgs* t, int n_tensors, int64_t B, int64_t H,
                        int64_t S, int D, int64_t stride_b, int64_t stride_h,
                        int64_t stride_s, const int8_t* signs, int64_t signs_stride_h,
                        int mode, float clip_ratio, int64_t S_cache, int64_t pos0,
                        hipStream_t stream);

}  // namespace quarot
