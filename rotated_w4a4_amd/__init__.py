"""rotated_w4a4_amd -- MI355X (gfx950) HIP kernels for QuaRot's online W4A4 path.

Python binding of the C ABI declared in ``include/quarot.h`` (library
``libquarot.so`` next to this file).  The binding only marshals arguments:
it checks dtypes, devices and shapes, passes raw device pointers and the
current HIP stream, and turns a negative status into an exception.  Every
step of the computation runs in the HIP kernels; there is no fallback.

Calls (same names as the C entry points, without the ``quarot_`` prefix):

* ``had_quant(x, signs, m, clip_ratio, had_m=None)`` -> (codes uint8 [rows, d/2],
  scales fp16 [rows])
* ``swiglu_had_quant(gate, up, signs, m, clip_ratio, had_m=None)`` -> (codes,
  scales) of the gated FFN product SiLU(gate) * up, formed in the same pass
* ``cross_head_had_quant(z, n_heads, clip_ratio)`` -> (codes, scales) of the
  attention output after the cross-head transform (out-projection input)
* ``w4a4_gemm(a_q, a_scale, b_q, b_scale, k)`` -> fp16 [M, N]
* ``kv_had_quant(k, v, signs, k_cache, k_scale, v_cache, v_scale, pos0)``
* ``kv_decode_attention(q, signs, k_cache, k_scale, v_cache, v_scale, max_len)``
  -> fp16 [B, Hq, 128] (one decode step over the int4 cache)
* ``kv_decode_attention_noalloc(...)``     -> the same without a workspace (the
  library's own scratch array; for callers that cannot allocate)
* ``kv_decode_workspace_bytes(B, Hq, Hkv, D, max_len)``
* ``hadamard_factor(m)``                  -> the library's Paley H_m (numpy int8)

Tensors are torch tensors on the current HIP device; torch provides device
memory and streams only.
"""

from ._lib import (QuarotError, cross_head_had_quant, had_quant, hadamard_factor,
                   kv_decode_attention, kv_decode_attention_noalloc, kv_decode_workspace_bytes,
                   kv_had_quant, lib, library_path, swiglu_had_quant, w4a4_gemm)

__all__ = ["QuarotError", "cross_head_had_quant", "had_quant", "hadamard_factor",
           "kv_decode_attention", "kv_decode_attention_noalloc", "kv_decode_workspace_bytes",
           "kv_had_quant", "lib", "library_path", "swiglu_had_quant", "w4a4_gemm"]
