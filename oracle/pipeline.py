"""End-to-end oracle of the online path: rotate+quant, weight prep, W4A4, KV.

* Activations ("QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs",
  paper-graph-ui summary, section 3.4 Stage 1b and Stage 2b): rotate each
  token by R, then per-token symmetric INT4, then pack.
* Weights (same page, Stage 1a "fuse Q into the weights" and Stage 2a; "QuaRot
  Guide", step 1 of "Deep Dive"): the same R is applied to each output
  channel's row of W [n_out x d] (W~ = W R^T), so X~ W~^T = X W^T; then one
  symmetric scale per output channel (max/7, round to nearest) and pack.
* Gated FFN producer (paper-graph-ui summary, section 3.4 "FFN Activation
  Rotation (Stage 1b)"): the down-projection's input is the SwiGLU product
  c = SiLU(A) * B, SiLU(t) = t * sigmoid(t) = t / (1 + exp(-t)), and the
  online Hadamard is applied to c; fusing it into its producer is the
  kernel improvement the page's section 6 names.  The product is formed in
  float64 and rotated without an intermediate fp16 rounding (the fused
  kernel never stores it).
* Out-projection input (same page, Stage 1c "Attention Value Projection
  Rotation"): the concatenated attention output Z gets the online cross-head
  transform Z (H_{n_h} (x) I_{d_h}) (no random signs: the head-wise factor
  and the out-projection weights absorb the rest of the rotation offline),
  then the per-token quantisation of Stage 2b feeds the INT4 out-projection.
* KV cache (same page, Stage 1d "online head-wise rotation after RoPE" and
  Stage 2c; "QuaRot Guide", step 4 of "Deep Dive"): each (batch, head,
  position) vector of head_dim values is rotated by the head-wise Hadamard and
  quantised as one group: symmetric (fp16 scale, int4 codes; the configured
  KV workload) or asymmetric (fp16 scale, fp16 integer zero point, uint4
  codes; Stage 2c's own quantiser, clip 0.95).
"""

from __future__ import annotations

import numpy as np

from .attention import cross_head
from .gemm import w4a4_reference
from .quant import pack_int4, pack_uint4, quantize_rows, quantize_rows_asym
from .rotate import rotate_rows

__all__ = ["had_quant", "prep_weights", "w4a4_linear", "kv_had_quant", "kv_had_quant_asym",
           "silu", "swiglu", "swiglu_had_quant", "cross_head_quant"]


def had_quant(x: np.ndarray, signs: np.ndarray, m: int = 1, clip_ratio: float = 1.0, hm=None):
    """Rotate+quant rows of x (hm: the small factor H_m, default Paley).

    Returns dict(x_rot float64, codes int8, packed uint8 [rows x d/2], scales fp16).
    """
    x_rot = rotate_rows(x, signs, m, hm)
    codes, scales = quantize_rows(x_rot, clip_ratio)
    return {"x_rot": x_rot, "codes": codes, "packed": pack_int4(codes), "scales": scales}


def prep_weights(w: np.ndarray, signs: np.ndarray, m: int = 1, hm=None):
    """Offline weight prep: W~ = W R^T, per-output-channel max/7 RTN, pack."""
    return had_quant(w, signs, m, clip_ratio=1.0, hm=hm)


def w4a4_linear(x: np.ndarray, w: np.ndarray, signs: np.ndarray, m: int = 1,
                clip_ratio: float = 1.0, hm=None):
    """The whole quantised linear layer: returns acts, weights, acc and y."""
    a = had_quant(x, signs, m, clip_ratio, hm)
    b = prep_weights(w, signs, m, hm)
    acc, y = w4a4_reference(a["codes"], a["scales"], b["codes"], b["scales"])
    return {"act": a, "wgt": b, "acc": acc, "y": y}


def kv_had_quant(t: np.ndarray, signs: np.ndarray, clip_ratio: float = 1.0):
    """Symmetric per-(b, h, s) group quantisation of a [B, H, S, D] tensor.

    Returns dict(x_rot [B,H,S,D] float64, codes int8, packed uint8 [B,H,S,D/2],
    scales fp16 [B,H,S]).
    """
    t = np.asarray(t)
    b, h, s, d = t.shape
    r = had_quant(t.reshape(-1, d), signs, 1, clip_ratio)
    return {
        "x_rot": r["x_rot"].reshape(b, h, s, d),
        "codes": r["codes"].reshape(b, h, s, d),
        "packed": r["packed"].reshape(b, h, s, d // 2),
        "scales": r["scales"].reshape(b, h, s),
    }


def kv_had_quant_asym(t: np.ndarray, signs: np.ndarray, clip_ratio: float = 0.95):
    """Asymmetric per-(b, h, s) group quantisation of a [B, H, S, D] tensor.

    Returns dict(x_rot float64, codes uint8 [B,H,S,D], packed uint8
    [B,H,S,D/2], scales fp16 [B,H,S], zeros int32 [B,H,S]).
    """
    t = np.asarray(t)
    b, h, s, d = t.shape
    x_rot = rotate_rows(t.reshape(-1, d), signs, 1)
    codes, scales, zeros = quantize_rows_asym(x_rot, clip_ratio)
    return {
        "x_rot": x_rot.reshape(b, h, s, d),
        "codes": codes.reshape(b, h, s, d),
        "packed": pack_uint4(codes).reshape(b, h, s, d // 2),
        "scales": scales.reshape(b, h, s),
        "zeros": zeros.reshape(b, h, s),
    }


def silu(t: np.ndarray) -> np.ndarray:
    """SiLU(t) = t / (1 + exp(-t)) in float64 (-0 where exp(-t) overflows)."""
    t = np.asarray(t, dtype=np.float64)
    with np.errstate(over="ignore"):
        return t / (1.0 + np.exp(-t))


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """The gated FFN product SiLU(gate) * up, elementwise, float64."""
    return silu(gate) * np.asarray(up, dtype=np.float64)


def swiglu_had_quant(gate: np.ndarray, up: np.ndarray, signs: np.ndarray, m: int = 1,
                     clip_ratio: float = 1.0, hm=None):
    """Rotate+quant of the gated product: had_quant(SiLU(gate) * up)."""
    return had_quant(swiglu(gate, up), signs, m, clip_ratio, hm)


def cross_head_quant(z: np.ndarray, n_heads: int, clip_ratio: float = 1.0):
    """Cross-head transform of each row of z [rows x n_heads*d_h] (heads
    concatenated, head h at lanes h*d_h .. h*d_h + d_h - 1), then per-token
    rotate+quant's quantiser.  Returns the same dict as had_quant."""
    z = np.asarray(z, dtype=np.float64)
    rows, d = z.shape
    if n_heads <= 0 or d % n_heads:
        raise ValueError("n_heads must divide the row length")
    z_rot = cross_head(z.reshape(rows, n_heads, d // n_heads)).reshape(rows, d)
    codes, scales = quantize_rows(z_rot, clip_ratio)
    return {"x_rot": z_rot, "codes": codes, "packed": pack_int4(codes), "scales": scales}
