"""Integer GEMM on INT4 codes and the per-token x per-channel dequantisation.

Definitions followed ("QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs",
paper-graph-ui summary, section 3.4 Stage 2b and "Kernel Implementation and
Hardware Efficiency"; "QuaRot Guide", step 3 of "Deep Dive"):

    acc[i, j] = sum_k qx[i, k] * qw[j, k]          (exact integer, INT32 on GPU)
    y[i, j]   = acc[i, j] * scale_x[i] * scale_w[j]  -> fp16

Reading: the summary casts acc to fp16 *before* scaling, which overflows once
|acc| > 65504 (|acc| reaches 64 * K).  The oracle instead forms
acc * scale_x * scale_w in float64 and rounds once to fp16 (round to nearest
even; beyond the fp16 range the result is +-inf, as a plain fp16 cast is).
"""

from __future__ import annotations

import numpy as np

__all__ = ["int_gemm", "int_gemm_exact", "dequant", "w4a4_reference"]


def int_gemm_exact(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc = qx @ qw^T with int64 accumulation (slow, the definition)."""
    return np.asarray(qx, dtype=np.int64) @ np.asarray(qw, dtype=np.int64).T


def int_gemm(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc = qx @ qw^T, exact, evaluated with float64 BLAS.

    Every product is an integer of magnitude <= 64 and every partial sum an
    integer of magnitude <= 64 * K < 2^53, so float64 represents each one
    exactly and the sum is exact in any order; the result is returned as int64.
    """
    qx = np.asarray(qx)
    qw = np.asarray(qw)
    if qx.shape[1] != qw.shape[1]:
        raise ValueError("inner dimensions differ")
    if 64 * qx.shape[1] >= 2 ** 53:
        raise ValueError("K too large for the exact float64 route")
    acc = qx.astype(np.float64) @ qw.astype(np.float64).T
    return acc.astype(np.int64)


def dequant(acc: np.ndarray, scale_x16: np.ndarray, scale_w16: np.ndarray) -> np.ndarray:
    """y = fp16(acc * scale_x[i] * scale_w[j]), product in float64, one rounding."""
    sx = np.asarray(scale_x16, dtype=np.float16).astype(np.float64)
    sw = np.asarray(scale_w16, dtype=np.float16).astype(np.float64)
    y = np.asarray(acc, dtype=np.float64) * sx[:, None] * sw[None, :]
    with np.errstate(over="ignore"):
        return y.astype(np.float16)


def w4a4_reference(qx, sx16, qw, sw16):
    """Integer GEMM + dequant: (acc int64, y fp16)."""
    acc = int_gemm(qx, qw)
    return acc, dequant(acc, sx16, sw16)
