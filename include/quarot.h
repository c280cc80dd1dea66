/*
 * quarot.h -- C ABI of the rotated W4A4 hot path for AMD Instinct MI355X (gfx950).
 *
 * The operations follow these pages (titles, with the section each call
 * follows):
 *   [S] "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs"
 *       (paper-graph-ui summary of arXiv 2404.00456)
 *   [G] "QuaRot Guide: Outlier-Free 4-Bit W4A4 LLM Quantization" (aifetchly blog)
 *   [V] the QuaRot paper-viz explainer (romaanj.github.io)
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer on the current HIP device,
 *     allocated and owned by the caller, except the small Hadamard factor
 *     had_m, which is read from HOST memory during the call.  The library
 *     allocates nothing, frees nothing and keeps no reference after
 *     returning.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     null stream) and the call returns without synchronising.  A kernel
 *     fault surfaces at the caller's next synchronisation.
 *   - fp16 means IEEE binary16 (stored as 16-bit words).  int4 codes are
 *     packed two per byte: element 2k in the low nibble of byte k, element
 *     2k+1 in the high nibble, each the 4-bit two's complement of a value
 *     in [-8, 7].
 *   - Return value: QUAROT_OK (0) or a negative status.  All argument checks
 *     run on the host before any HIP call, so a rejected call touches
 *     neither the GPU nor the stream.  quarot_last_error() returns a
 *     thread-local text with the detail of the last failure on this thread.
 *   - Calls are re-entrant; the library holds no mutable global state apart
 *     from a once-initialised per-device property cache.
 */
#ifndef QUAROT_H
#define QUAROT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  QUAROT_OK = 0,
  QUAROT_ERR_INVALID = -1,     /* null required pointer, bad size, bad stride, bad clip */
  QUAROT_ERR_UNSUPPORTED = -2, /* shape or mode outside what the kernels implement */
  QUAROT_ERR_MISALIGNED = -3,  /* pointer or stride alignment requirement violated */
  QUAROT_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
};

/*
 * Fused randomized Hadamard rotation + per-token symmetric INT4 quantisation.
 *
 * Follows [S] section 3.4 Stage 1a (randomized Hadamard R = H diag(s), and
 * H_d = H_{2^n} (x) H_m with a known Hadamard matrix H_m when d is not a
 * power of two), Stage 1b (online Hadamard before the down-projection),
 * Stage 2b (per-token symmetric scale clip * max|x| / 7) and "Kernel
 * Implementation and Hardware Efficiency" (quantise per token, pack two INT4
 * per byte); [G] section "2. Why Randomized Walsh-Hadamard Transforms" and
 * step 2 of "Deep Dive" (round to nearest, clip to [-8, 7]).
 *
 * For every row r of x (fp16 [rows x d], row stride ld_x elements):
 *   x~      = (H_{2^n} (x) H_m) diag(signs) x_r / sqrt(d)      (fp32 arithmetic)
 *   S_r     = fp16(clip_ratio * max(max_j |x~_j|, 1e-5) / 7)
 *   q_j     = clamp(rint(x~_j / S_r), -8, 7)                     (ties to even)
 * and writes q packed into q_out (uint8 [rows x d/2], row stride ld_q bytes)
 * and S_r into scale_out (fp16 [rows]).  The Kronecker index of element j
 * is j = a*m + b: H_m mixes the contiguous group b (row b of had_m weights
 * column c: y[a*m + b] = sum_c had_m[b*m + c] x[a*m + c]), H_{2^n} (the
 * Sylvester matrix, entry (i, j) = (-1)^popcount(i & j)) mixes a.
 *
 * Arguments:
 *   x          fp16 [rows x d], 16-byte aligned, ld_x >= d, ld_x % 8 == 0.
 *   signs      int8 [d] of +1/-1, or NULL for all +1.
 *   m          1, or a multiple of 4 up to 32: the order of the small
 *              Hadamard factor; d = 2^n * m.
 *   had_m      HOST memory: int8 [m x m] row-major, entries +1/-1, with
 *              had_m had_m^T = m I (checked).  NULL iff m == 1.  It is read
 *              during the call and handed to the kernels by value; the
 *              library keeps no reference.  quarot_hadamard_factor() returns
 *              the Paley matrices of order 12 and 28 the configs use; offline
 *              weight preparation must use the same matrix as the activations.
 *   clip_ratio in (0, 1].  1.0 gives S = max|x~| / 7.
 *   q_out      uint8 [rows x ld_q], 16-byte aligned, ld_q >= d/2, ld_q % 16 == 0.
 *   scale_out  fp16 [rows], 2-byte aligned.
 *   x_rot_out  optional fp32 [rows x d] (dense) receiving x~ for inspection;
 *              NULL in production (it adds 4*d bytes of traffic per row).
 * Supported: rows >= 0 (0 is a no-op), d = 2^n * m with d % 32 == 0 and
 * d <= 32768.  Non-finite inputs are outside the contract.
 * Errors: INVALID for bad sizes, strides, clip, a missing required pointer,
 * had_m given with m == 1 or missing with m > 1, or had_m not a Hadamard
 * matrix; UNSUPPORTED for other m or d; MISALIGNED as stated.
 */
int quarot_had_quant(const void* x, int64_t rows, int64_t d, int64_t ld_x,
                     const int8_t* signs, int32_t m, const int8_t* had_m, float clip_ratio,
                     uint8_t* q_out, int64_t ld_q, void* scale_out,
                     float* x_rot_out, void* stream);

/*
 * The gated FFN product fused into rotate+quant: the row that is rotated and
 * quantised is c = SiLU(gate) * up, formed in the same pass, so the product
 * never travels through HBM.
 *
 * Follows [S] section 3.4 "FFN Activation Rotation (Stage 1b)" (the online
 * Hadamard is applied to the SwiGLU output (SiLU(A) * B) H right before the
 * down-projection) and section 6 "Limitations and Trade-offs" (fusing the
 * quantisation into the neighbouring kernels is the open kernel
 * improvement); the rotation and quantiser are those of quarot_had_quant.
 *
 * For every row r:
 *   c_j   = SiLU(gate_rj) * up_rj,   SiLU(t) = t / (1 + exp(-t))   (fp32)
 *   then x~, S_r and the codes exactly as quarot_had_quant with c in place
 *   of x.  The product is not rounded to fp16 before the rotation: the
 *   kernels keep about 22 significant bits of it (fp32 rotation input).
 *
 * Arguments:
 *   gate, up   fp16 [rows x d] each, 16-byte aligned, row strides ld_gate,
 *              ld_up >= d and multiples of 8 (a fused gate_up projection
 *              output [rows x 2d] is gate = p, up = p + d, both strides 2d).
 *   everything else as quarot_had_quant; x_rot_out receives the rotated
 *   product.  Products beyond the fp16 range (|c| > 65504) are outside the
 *   contract.
 */
int quarot_swiglu_had_quant(const void* gate, const void* up, int64_t rows, int64_t d,
                            int64_t ld_gate, int64_t ld_up, const int8_t* signs, int32_t m,
                            const int8_t* had_m, float clip_ratio, uint8_t* q_out, int64_t ld_q,
                            void* scale_out, float* x_rot_out, void* stream);

/*
 * Cross-head transform + per-token symmetric INT4 quantisation of the
 * attention output (the input of the INT4 out-projection).
 *
 * Follows [S] section 3.4 Stage 1c (the head-wise factor I_{n_h} (x) H_{d_h}
 * of the full Hadamard is folded into W_v and W_out offline; the online block
 * after attention computes Z <- Z (H_{n_h} (x) I_{d_h}), a Walsh-Hadamard
 * transform of length n_h over the head index for every head-dim lane) and
 * Stage 2b (per-token scale clip * max|z~| / 7).  No random signs: the
 * out-projection weights absorb the same plain Hadamard offline.
 *
 * For every row r of z (fp16 [rows x n_heads*head_dim], head h at elements
 * h*head_dim .. h*head_dim + head_dim - 1, row stride ld_z elements):
 *   z~[a*head_dim + c] = sum_a' H[a', a] z[a'*head_dim + c] / sqrt(n_heads)
 * with H the Sylvester matrix H[i][j] = (-1)^popcount(i & j), then S_r and
 * the codes exactly as quarot_had_quant (fp32 arithmetic, ties to even).
 *
 * Arguments:
 *   z          fp16, 4-byte aligned, ld_z >= n_heads*head_dim, ld_z even.
 *   n_heads    a power of two, 1 .. 64 (1 = quantisation only).
 *   head_dim   128.
 *   clip_ratio in (0, 1].
 *   q_out      uint8 [rows x ld_q], ld_q >= n_heads*head_dim/2.
 *   scale_out  fp16 [rows], 2-byte aligned.
 *   z_rot_out  optional fp32 [rows x n_heads*head_dim] (dense, 8-byte
 *              aligned) receiving z~; NULL in production.
 * Errors: INVALID for negative rows, bad strides, clip or a missing required
 * pointer; UNSUPPORTED for other head_dim or n_heads; MISALIGNED as stated.
 * rows == 0 is a no-op.  Non-finite inputs are outside the contract.
 */
int quarot_cross_head_had_quant(const void* z, int64_t rows, int64_t n_heads, int64_t head_dim,
                                int64_t ld_z, float clip_ratio, uint8_t* q_out, int64_t ld_q,
                                void* scale_out, float* z_rot_out, void* stream);

/*
 * W4A4 GEMM with INT32 accumulation and the per-token x per-channel dequant.
 *
 * Follows [S] section 3.4 Stage 2b (dequantised output
 * Y_ij = acc_ij * scale_x[i] * scale_w[j]) and "Kernel Implementation and
 * Hardware Efficiency" (INT4 x INT4 GEMM of packed activations against
 * offline-packed weights, INT32 accumulator, dequant to FP16); [G] step 3
 * of "Deep Dive".
 *
 *   acc[i][j] = sum_k a[i][k] * b[j][k]           exact, int32
 *   c[i][j]   = fp16(float(acc[i][j]) * a_scale[i] * b_scale[j])
 * (computed in fp32, then rounded to fp16 with ties to even;
 * beyond the fp16 range it saturates to +-inf).
 *
 * Arguments:
 *   a_q        packed int4 activations, uint8 [M x lda], K-contiguous rows,
 *              16-byte aligned, lda >= K/2, lda % 16 == 0.
 *   a_scale    fp16 [M] per-token scales.
 *   b_q        packed int4 weights, uint8 [N x ldb] (one row per output
 *              channel), same alignment rules as a_q.
 *   b_scale    fp16 [N] per-output-channel scales.
 *   c          fp16 [M x ldc] output, ldc >= N, 2-byte aligned.
 *   acc_out    optional int32 [M x ld_acc] receiving acc (ld_acc >= N);
 *              NULL in production.
 * Supported: M, N >= 0 (0 is a no-op), K > 0 with K % 32 == 0 and
 * K <= 65536 (so 256 * |acc| <= 256 * 64 K fits in int32); M, N < 2^31,
 * else UNSUPPORTED (as is a grid of 2^32 or more work items, which takes
 * over 10^12 outputs).
 */
int quarot_w4a4_gemm(const uint8_t* a_q, int64_t lda, const void* a_scale,
                     const uint8_t* b_q, int64_t ldb, const void* b_scale,
                     int64_t M, int64_t N, int64_t K,
                     void* c, int64_t ldc, int32_t* acc_out, int64_t ld_acc,
                     void* stream);

/*
 * Head-wise Hadamard rotation + INT4 quantisation of K and V into the cache.
 *
 * Follows [S] section 3.4 Stage 1d (keys rotated head-wise by
 * I_{n_h} (x) H_{d_h} after RoPE, post-RoPE caching), Stage 1c (values
 * rotated head-wise), Stage 2c (one quantisation group per head vector of
 * 128 values) and the "Append" routine of "Kernel Implementation and
 * Hardware Efficiency" (quantise the new keys/values and append them to the
 * cache); [G] step 4 of "Deep Dive".
 *
 * For every (b, h, s) with 0 <= s < S, the D values
 * t[b][h][s][:] (element (b,h,s,i) at t + b*stride_b + h*stride_h +
 * s*stride_s + i) are rotated by diag(signs_h) then the Sylvester H_D / sqrt(D)
 * and quantised as one group, with the code row written to cache position
 * p = pos0 + s:
 *   t_q    [B x H x S_cache x D/2] uint8, contiguous, row (b,h,p)
 *   t_scale[B x H x S_cache]       fp16, contiguous
 *   t_zero [B x H x S_cache]       fp16, contiguous (mode 1 only).
 * mode 0 (symmetric, the configured cache workload): exactly like
 *   quarot_had_quant: S = fp16(clip * max(max|x~|, 1e-5) / 7),
 *   q = clamp(rint(x~ / S), -8, 7) as two's complement nibbles.
 * mode 1 (asymmetric, [S] Stage 2c's own KV quantiser; the pages use
 *   clip 0.95): alpha_min = clip * min x~, alpha_max = clip * max x~,
 *   S = fp16(max(alpha_max - alpha_min, 1e-5) / 15),
 *   z = clamp(rint(-alpha_min / S), -1024, 1024) stored as fp16 (exact),
 *   q = clamp(rint(x~ / S) + z, 0, 15) as unsigned nibbles; x^ = S (q - z).
 * In both modes element 2k goes to the low nibble of byte k; the decisions
 * are taken in fp32 from the stored fp16 scale.
 *
 * Arguments:
 *   k, v         fp16 inputs; either may be NULL (that tensor is skipped),
 *                not both.  16-byte aligned; strides in elements, each a
 *                multiple of 8 and >= 0.
 *   D            head dimension: 32, 64, 128 or 256.
 *   signs        int8 +1/-1; head h uses signs + h*signs_stride_h (stride 0:
 *                one vector shared by all heads).  NULL = all +1.
 *   mode         0 = symmetric, 1 = asymmetric with a zero point.
 *   clip_ratio   in (0, 1].
 *   k_q/v_q      16-byte aligned cache code buffers; k_scale/v_scale fp16.
 *   k_zero/v_zero  fp16, 2-byte aligned; required in mode 1 for every tensor
 *                given, ignored in mode 0.
 *   S_cache, pos0  cache length and first position written;
 *                0 <= pos0 and pos0 + S <= S_cache.
 *   k_rot_out, v_rot_out  optional fp32 [B x H x S x D] (dense, indexed by
 *                the input position s, 16-byte aligned) receiving the rotated
 *                groups x~ for inspection; NULL in production.  Ignored for a
 *                tensor that is not given.
 * Errors: INVALID for bad sizes, mode, clip or missing buffers;
 * UNSUPPORTED for other D or B*H*S >= 2^31; MISALIGNED as stated.
 */
int quarot_kv_had_quant(const void* k, const void* v,
                        int64_t B, int64_t H, int64_t S, int64_t D,
                        int64_t stride_b, int64_t stride_h, int64_t stride_s,
                        const int8_t* signs, int64_t signs_stride_h,
                        int32_t mode, float clip_ratio,
                        uint8_t* k_q, void* k_scale, void* k_zero,
                        uint8_t* v_q, void* v_scale, void* v_zero,
                        int64_t S_cache, int64_t pos0, float* k_rot_out, float* v_rot_out,
                        void* stream);

/*
 * One decode step of attention over the INT4 cache written by
 * quarot_kv_had_quant, with the query rotation and, optionally, the
 * cross-head transform.
 *
 * Follows [S] section 3.4 Stage 1d (the new query is rotated head-wise by
 * the same Hadamard as the cached keys, after RoPE, so q k^T is unchanged;
 * P = softmax(q K^T / sqrt(d_h))), Stage 2c (the decode-time list: rotate
 * the query, load the quantised keys and values of all previous positions,
 * dequantise every group on the fly, attend) and Stage 1c (the online
 * cross-head transform Z <- Z (H_{n_h} (x) I_{d_h}) on the concatenated
 * attention output).
 *
 * For batch row b and query head j (KV head h = j / (Hq / Hkv): consecutive
 * query heads share a KV head), with L = min(lengths[b], max_len) (max_len
 * when lengths is NULL) and positions p < L:
 *   q~ = H_128 diag(signs_h) q[b][j] / sqrt(128)          (fp32)
 *   k^_p = S_p * c_p  (mode 0)  or  S_p * (u_p - z_p)  (mode 1), likewise v^_p
 *   out[b][j] = sum_p softmax_p(sm_scale * q~ . k^_p) v^_p
 * in fp32-class arithmetic (scores and P V on fp16 matrix cores with the
 * fp32 operand split into fp16 high and low parts).  The output stays in the
 * rotated basis of the values.  With cross_head != 0 the Hq outputs of each
 * batch row are then mixed by the normalised Sylvester H_Hq over the head
 * index: out'[b][a][d] = sum_a' H[a][a'] out[b][a'][d] / sqrt(Hq).  A row
 * with L = 0 gives 0.
 *
 * Arguments:
 *   q            fp16 [B x Hq x 128], contiguous, 16-byte aligned (post-RoPE
 *                queries, not rotated).
 *   signs        int8 +1/-1, KV head h uses signs + h*signs_stride_h; must be
 *                what the cache was written with.  NULL = all +1.
 *   mode         0 = symmetric cache, 1 = zero-point cache (k_zero, v_zero
 *                required).
 *   k_q, v_q     uint8 [B x Hkv x S_cache x 64], 16-byte aligned;
 *   k_scale, v_scale, k_zero, v_zero  fp16 [B x Hkv x S_cache].
 *   D            head dimension; 128 only.
 *   Hq, Hkv      Hq a multiple of Hkv, Hq / Hkv <= 8.
 *   max_len      1 <= max_len <= S_cache (and <= 2^24): positions attended
 *                at most.
 *   lengths      optional int32 [B] device array of per-row lengths (values
 *                above max_len are clamped to it, negative ones to 0).
 *   sm_scale     softmax scale, finite and > 0 (1/sqrt(128) in the pages).
 *   cross_head   0 or 1; 1 needs Hq a power of two <= 256.
 *   out          fp16 [B x Hq x 128], 2-byte aligned; out_f32 optional fp32
 *                copy (same layout, 4-byte aligned) for parity checks.
 *   workspace    device scratch of at least
 *                quarot_kv_decode_workspace_bytes(B, Hq, Hkv, D, max_len)
 *                bytes, 16-byte aligned, owned by the caller; its contents
 *                on entry do not matter.  Calls that share a workspace must
 *                be ordered (one stream).
 * Errors: INVALID for bad sizes, mode, scale, missing buffers or a short
 * workspace; UNSUPPORTED for D != 128, Hq / Hkv > 8, max_len > 2^24,
 * B * Hkv >= 2^24, or cross_head with Hq not a power of two <= 256;
 * MISALIGNED as stated.
 */
int quarot_kv_decode_attention(const void* q, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                               const int8_t* signs, int64_t signs_stride_h, int32_t mode,
                               const uint8_t* k_q, const void* k_scale, const void* k_zero,
                               const uint8_t* v_q, const void* v_scale, const void* v_zero,
                               int64_t S_cache, int64_t max_len, const int32_t* lengths,
                               float sm_scale, int32_t cross_head,
                               void* out, float* out_f32,
                               void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Allocation-free variant of quarot_kv_decode_attention, for callers that
 * cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 *
 * Arguments, results and errors as quarot_kv_decode_attention without the
 * workspace.  The per-split partials go to a scratch array inside the
 * library: QUAROT_DECODE_SCRATCH_BYTES per GPU, a file-scope device array
 * that each GPU the library runs on holds until the process ends.  A call
 * whose sizes need more (quarot_kv_decode_workspace_bytes() above the limit)
 * is rejected with QUAROT_ERR_UNSUPPORTED before any launch.  The call makes
 * no allocation (no hipMalloc, hipFree or allocating library routine); its
 * first call on a device looks up that device's scratch address.  Every call
 * on one GPU shares that GPU's array, which keeps the last call's contents
 * (no call depends on them: every partial read is written first in the same
 * call), so calls that overlap on one GPU (other streams, other threads)
 * race: order them on one stream.
 */
#define QUAROT_DECODE_SCRATCH_BYTES (8 * 1024 * 1024)

int quarot_kv_decode_attention_noalloc(const void* q, int64_t B, int64_t Hq, int64_t Hkv,
                                       int64_t D, const int8_t* signs, int64_t signs_stride_h,
                                       int32_t mode, const uint8_t* k_q, const void* k_scale,
                                       const void* k_zero, const uint8_t* v_q,
                                       const void* v_scale, const void* v_zero, int64_t S_cache,
                                       int64_t max_len, const int32_t* lengths, float sm_scale,
                                       int32_t cross_head, void* out, float* out_f32,
                                       void* stream);

/*
 * Host-only: bytes of workspace quarot_kv_decode_attention needs for these
 * sizes (per position split: the running max, softmax sum and unnormalised
 * output of every query head).  Returns a negative status for sizes the
 * entry point would reject.  Makes no HIP call.
 */
int64_t quarot_kv_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                         int64_t max_len);

/*
 * Host-only: copy one of the library's Paley type-I Hadamard matrices
 * (entries +1/-1, row-major int8 [m x m], HOST memory of m*m bytes), for a
 * caller to pass as had_m.  m = 1 gives [1]; 12 and 28 give the Paley
 * matrices for q = 11 and q = 27 ([S] Stage 1a takes any known Hadamard
 * matrix of order m; [V] builds width 12288 with a Paley block of 12).  Offline weight
 * preparation must rotate with the same matrix as the activations.  Makes
 * no HIP call.
 */
int quarot_hadamard_factor(int32_t m, int8_t* out_host);

/* Static text for a status code (never NULL). */
const char* quarot_status_string(int status);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char* quarot_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QUAROT_H */
