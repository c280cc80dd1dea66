"""Symmetric INT4 round-to-nearest quantisation and nibble packing.

Definitions followed:

* "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
  summary), section 3.4 "Quantization Scheme (Stage 2)":
  - Stage 2a (weights, offline): one symmetric scale per output channel,
    s = max|w| / (2^(b-1) - 1) = max|w| / 7 for b = 4.
  - Stage 2b (activations, online): one symmetric scale per token,
    s = clip * max_j |x_j| / 7 (the summary uses clip 0.9).
  - "Kernel Implementation and Hardware Efficiency": quantise per token, then
    pack two INT4 values per byte.
* "QuaRot Guide: Outlier-Free 4-Bit W4A4 LLM Quantization", section "3. The
  Collapse of Naive W4A4" and step 2 of "Deep Dive": x_q = clip(round(x / S),
  -8, 7) with S = max|x| / 7, i.e. clip = 1.0; its code clamps the absolute
  maximum below by 1e-5 and rounds half to even.

Readings taken where the pages leave a step open (each is listed with the
other readings of the pages in the design notes):

* The scale is stored in fp16 and the codes are computed from the stored
  (fp16-rounded) scale, so stored scales and codes always agree.
* The rounding decision x / S -> integer is the definition evaluated exactly:
  the float64 rotated value divided by the stored scale widened to float64,
  rounded half to even (``np.rint``).  A kernel that rotates in fp32 can land
  on the other side of a rounding boundary on a few elements; that is what
  the code tolerance of the parity tests measures.
* Nibble order: element 2k goes to the low nibble of byte k, element 2k+1 to
  the high nibble; each nibble is the 4-bit two's complement of the code.
* An all-zero row keeps the 1e-5 floor: its scale is fp16(clip * 1e-5 / 7)
  and its codes are all zero.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "ZMAX",
    "asym_params",
    "asym_codes",
    "quantize_rows_asym",
    "pack_uint4",
    "unpack_uint4",
    "QMIN",
    "QMAX",
    "ABSMAX_FLOOR",
    "row_scales",
    "codes_from_scales",
    "quantize_rows",
    "pack_int4",
    "unpack_int4",
]

QMIN = -8
QMAX = 7
ABSMAX_FLOOR = 1e-5


def row_scales(x_rot: np.ndarray, clip_ratio: float = 1.0) -> np.ndarray:
    """Per-row symmetric scale, fp16: S = fp16(clip * max(max_j |x_j|, 1e-5) / 7)."""
    if not (0.0 < clip_ratio <= 1.0):
        raise ValueError("clip_ratio must be in (0, 1]")
    a = np.max(np.abs(np.asarray(x_rot, dtype=np.float64)), axis=1)
    a = np.maximum(a, ABSMAX_FLOOR)
    return (clip_ratio * a / QMAX).astype(np.float16)


def codes_from_scales(x_rot: np.ndarray, scales16: np.ndarray) -> np.ndarray:
    """q = clamp(rint(x / float64(S)), -8, 7), one scale per row (int8)."""
    x64 = np.asarray(x_rot, dtype=np.float64)
    s64 = np.asarray(scales16, dtype=np.float16).astype(np.float64)[:, None]
    r = np.rint(x64 / s64)  # float64 division, ties to even
    return np.clip(r, QMIN, QMAX).astype(np.int8)


def quantize_rows(x_rot: np.ndarray, clip_ratio: float = 1.0):
    """Per-row symmetric INT4: returns (codes int8 [rows x d], scales fp16 [rows])."""
    s = row_scales(x_rot, clip_ratio)
    return codes_from_scales(x_rot, s), s


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte: byte k = (q[2k] & 0xF) | ((q[2k+1] & 0xF) << 4)."""
    q = np.asarray(codes, dtype=np.int64)
    if q.shape[-1] % 2:
        raise ValueError("need an even number of codes per row")
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4 (int8 codes in [-8, 7])."""
    b = np.asarray(packed, dtype=np.int64)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ---------------------------------------------------------------------------
# Asymmetric per-group INT4 (the KV cache's own quantiser)
#
# "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
# summary), section 3.4 Stage 2c: per-group asymmetric quantisation with a
# scale and a zero point, s = (alpha_max - alpha_min) / (2^b - 1), the range
# taken with a clipping ratio of 0.95, group = the 128 values of one head.
# The page's zero-point formula mixes units (it subtracts round(alpha_min /
# s) from a value in real units); the reading used here is the textbook
# uint4 form that the rest of the passage describes:
#   alpha_min = clip * min(x),  alpha_max = clip * max(x)
#   S = fp16(max(alpha_max - alpha_min, 1e-5) / 15)
#   z = clamp(rint(-alpha_min / S), -ZMAX, ZMAX)          (integer zero point)
#   q = clamp(rint(x / S) + z, 0, 15)                     (uint4 code)
#   x_hat = S * (q - z)
# with the same precision conventions as the symmetric quantiser: S is the
# stored fp16 scale (rounded once from the float64 range); alpha, the
# zero-point division and x / S are float64 with ties to even; z is kept
# within +-ZMAX so it is exactly representable in the fp16 it is stored in.
# ---------------------------------------------------------------------------

ZMAX = 1024
UQMAX = 15


def asym_params(x_rot: np.ndarray, clip_ratio: float = 0.95):
    """Per-row (scale fp16, zero point int32) of the asymmetric quantiser."""
    if not (0.0 < clip_ratio <= 1.0):
        raise ValueError("clip_ratio must be in (0, 1]")
    x64 = np.asarray(x_rot, dtype=np.float64)
    c = float(clip_ratio)
    amin = c * x64.min(axis=1)
    amax = c * x64.max(axis=1)
    rng = np.maximum(amax - amin, ABSMAX_FLOOR)
    s16 = (rng / UQMAX).astype(np.float16)
    z = np.rint(-amin / s16.astype(np.float64))
    z = np.clip(z, -ZMAX, ZMAX).astype(np.int32)
    return s16, z


def asym_codes(x_rot: np.ndarray, scales16: np.ndarray, zeros: np.ndarray) -> np.ndarray:
    """q = clamp(rint(x / float64(S)) + z, 0, 15), one (S, z) per row (uint8)."""
    x64 = np.asarray(x_rot, dtype=np.float64)
    s64 = np.asarray(scales16, dtype=np.float16).astype(np.float64)[:, None]
    r = np.rint(x64 / s64) + np.asarray(zeros, dtype=np.float64)[:, None]
    return np.clip(r, 0, UQMAX).astype(np.uint8)


def quantize_rows_asym(x_rot: np.ndarray, clip_ratio: float = 0.95):
    """Per-row asymmetric uint4: returns (codes uint8, scales fp16, zeros int32)."""
    s, z = asym_params(x_rot, clip_ratio)
    return asym_codes(x_rot, s, z), s, z


def pack_uint4(codes: np.ndarray) -> np.ndarray:
    """Two uint4 codes per byte: byte k = q[2k] | (q[2k+1] << 4)."""
    q = np.asarray(codes, dtype=np.int64)
    if q.shape[-1] % 2:
        raise ValueError("need an even number of codes per row")
    if q.min(initial=0) < 0 or q.max(initial=0) > UQMAX:
        raise ValueError("uint4 codes must be in [0, 15]")
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def unpack_uint4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_uint4 (uint8 codes in [0, 15])."""
    b = np.asarray(packed, dtype=np.int64)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = (b >> 4) & 0xF
    return out
