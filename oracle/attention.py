"""Decode-step attention over the INT4 KV cache, and the cross-head rotation.

Definitions followed:

* "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
  summary), section 3.4 "Key and Query Rotation (Stage 1d)": queries and keys
  are both rotated head-wise after RoPE, Q <- RoPE(X W_q) (I (x) H_{d_h}), so
  the scores Q_h K_h^T are unchanged; at decode the single new query is
  rotated online while the keys in the cache were rotated when written.
  P_h = softmax(Q_h K_h^T / sqrt(d_h)) with the causal mask.
* Same page, "KV Cache Quantization (Stage 2c)", the decode-time list: rotate
  the query head-wise, load the quantised keys and values of all previous
  positions, dequantise each group on the fly, compute the attention, append.
* Same page, "Attention Value Projection Rotation (Stage 1c)": the attention
  output Z (heads concatenated, before the output projection) gets the online
  cross-head transform Z <- Z (H_{n_h} (x) I_{d_h}), a Walsh-Hadamard transform
  of length n_h over the head index for every (position, head-dim) pair.

Readings taken where the pages leave a step open:

* The query gets exactly the rotation the cache's keys got,
  R = H_{d_h} diag(s) / sqrt(d_h) (signs of its KV head), so q~ . k~ = q . k.
* Grouped-query attention: query head j reads KV head j // (H_q / H_kv)
  (consecutive query heads share one KV head).
* Dequantisation: symmetric k^ = S * q; asymmetric k^ = S * (u - z), the
  inverse of the cache quantiser (the pages' "s * v + z" is taken as that).
* The output stays in the rotated basis of the values (the head-wise H folds
  into W_out offline, Stage 1c); the cross-head transform, when asked for, is
  the normalised Sylvester H_{H_q} applied over the head index.
* A batch row whose valid length is 0 attends to nothing: its output is 0.

Everything is float64.  The attention itself is the textbook formula with a
max-subtracted softmax; no blocking or online rescaling.
"""

from __future__ import annotations

import math

import numpy as np

from .hadamard import sylvester
from .quant import unpack_int4, unpack_uint4
from .rotate import rotate_rows

__all__ = ["dequant_cache", "rotate_heads", "attend", "cross_head", "decode_attention"]


def dequant_cache(packed: np.ndarray, scales: np.ndarray, zeros=None, mode: int = 0) -> np.ndarray:
    """Cache groups [..., D/2] uint8 + fp16 scales [...] (+ fp16 zeros) -> float64 [..., D]."""
    packed = np.asarray(packed)
    lead = packed.shape[:-1]
    flat = packed.reshape(-1, packed.shape[-1])
    s = np.asarray(scales, dtype=np.float16).astype(np.float64).reshape(-1, 1)
    if mode == 0:
        vals = unpack_int4(flat).astype(np.float64) * s
    elif mode == 1:
        z = np.asarray(zeros, dtype=np.float16).astype(np.float64).reshape(-1, 1)
        vals = (unpack_uint4(flat).astype(np.float64) - z) * s
    else:
        raise ValueError("mode must be 0 (symmetric) or 1 (asymmetric)")
    return vals.reshape(*lead, -1)


def rotate_heads(q: np.ndarray, signs: np.ndarray, n_kv: int) -> np.ndarray:
    """q [B, Hq, D] -> R q per head, with the signs of the head's KV head.

    ``signs`` is [D] (shared by every head) or [H_kv, D].
    """
    q = np.asarray(q)
    b, hq, d = q.shape
    group = hq // n_kv
    signs = np.asarray(signs)
    out = np.empty((b, hq, d), dtype=np.float64)
    for j in range(hq):
        s = signs if signs.ndim == 1 else signs[j // group]
        out[:, j, :] = rotate_rows(q[:, j, :], s)
    return out


def attend(q_rot: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, lengths,
           sm_scale: float) -> np.ndarray:
    """softmax(q k^T * sm_scale) v for every (batch, query head).

    q_rot [B, Hq, D]; k_hat, v_hat [B, H_kv, S, D]; lengths [B] (positions
    0 .. len-1 are attended).  Returns float64 [B, Hq, D].
    """
    b, hq, d = q_rot.shape
    n_kv = k_hat.shape[1]
    group = hq // n_kv
    out = np.zeros((b, hq, d), dtype=np.float64)
    for bi in range(b):
        n = int(lengths[bi])
        if n <= 0:
            continue
        for j in range(hq):
            kv = j // group
            k = k_hat[bi, kv, :n, :]
            v = v_hat[bi, kv, :n, :]
            scores = (k @ q_rot[bi, j, :]) * sm_scale
            p = np.exp(scores - scores.max())
            out[bi, j, :] = (p @ v) / p.sum()
    return out


def cross_head(z: np.ndarray) -> np.ndarray:
    """Z (H_{Hq} (x) I_D) / sqrt(Hq) on z [B, Hq, D]: out[b, a, d] = sum_a' z[b, a', d] H[a', a]."""
    z = np.asarray(z, dtype=np.float64)
    hq = z.shape[1]
    h = sylvester(hq).astype(np.float64)
    return np.einsum("bkd,ka->bad", z, h) / math.sqrt(hq)


def decode_attention(q: np.ndarray, signs: np.ndarray, cache: dict, lengths, sm_scale=None,
                     mode: int = 0, cross: bool = False) -> np.ndarray:
    """One decode step: rotate q head-wise, dequantise the cache, attend.

    ``cache`` holds k_q, k_scale, v_q, v_scale ([B, H_kv, S, D/2] uint8 and
    [B, H_kv, S] fp16) and, for mode 1, k_zero, v_zero.  Returns float64
    [B, Hq, D] (cross-head transformed when ``cross``).
    """
    k_hat = dequant_cache(cache["k_q"], cache["k_scale"], cache.get("k_zero"), mode)
    v_hat = dequant_cache(cache["v_q"], cache["v_scale"], cache.get("v_zero"), mode)
    d = k_hat.shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    q_rot = rotate_heads(q, signs, k_hat.shape[1])
    out = attend(q_rot, k_hat, v_hat, lengths, sm_scale)
    return cross_head(out) if cross else out
