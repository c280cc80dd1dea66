"""Randomized Hadamard rotation of rows, in float64.

Definition followed ("QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs",
paper-graph-ui summary, section 3.4 Stage 1a; "QuaRot Guide", section "2. Why
Randomized Walsh-Hadamard Transforms (RHT) Disperse Outliers"):

    R = H_d * diag(s) / sqrt(d),     H_d = H_{2^n} (x) H_m,

acting on column vectors, so a row x becomes x~ = R x (rows: X~ = X R^T).
Signs are applied first, then H_d.  The Kronecker index of entry (a, b) is
a * m + b: b runs over a contiguous group of m and is mixed by H_m, a has
stride m and is mixed by H_{2^n}.

Applying H_{2^n} (x) H_m is done by its defining entrywise formula
(H_{2^n} (x) H_m)[(a,b),(a',b')] = H_{2^n}[a,a'] * H_m[b,b'], i.e. one matrix
product over b' and one over a' -- no butterflies.  ``dense_rotation`` builds
the full d x d matrix for small d.
"""

from __future__ import annotations

import math

import numpy as np

from .hadamard import hadamard_m, sylvester

__all__ = ["rotate_rows", "dense_rotation", "split_d"]


def split_d(d: int, m: int) -> int:
    """Return n with d = 2^n * m, or raise."""
    if m < 1 or d % m:
        raise ValueError(f"d = {d} is not a multiple of m = {m}")
    p = d // m
    if p & (p - 1):
        raise ValueError(f"d / m = {p} is not a power of two")
    return p.bit_length() - 1


def _factor(m: int, hm) -> np.ndarray:
    """H_m as float64: the given matrix, or the Paley matrix of order m."""
    if hm is None:
        return hadamard_m(m).astype(np.float64)
    h = np.asarray(hm)
    if h.shape != (m, m):
        raise ValueError(f"hm must be [{m} x {m}]")
    return h.astype(np.float64)


def dense_rotation(d: int, signs: np.ndarray, m: int = 1, hm=None) -> np.ndarray:
    """The full rotation R = (H_{2^n} (x) H_m) diag(s) / sqrt(d), float64 [d x d]."""
    n = split_d(d, m)
    h = np.kron(sylvester(1 << n).astype(np.float64), _factor(m, hm))
    return h * signs.astype(np.float64)[None, :] / math.sqrt(d)


def rotate_rows(x: np.ndarray, signs: np.ndarray, m: int = 1, hm=None,
                chunk_rows: int = 256) -> np.ndarray:
    """x~ = R x for every row of x (any real dtype in, float64 out).  hm: the
    small factor H_m (default: the Paley matrix of order m)."""
    x = np.asarray(x)
    rows, d = x.shape
    n = split_d(d, m)
    p = 1 << n
    h2 = sylvester(p).astype(np.float64)
    hm = _factor(m, hm)
    s = signs.astype(np.float64)
    inv = 1.0 / math.sqrt(d)
    out = np.empty((rows, d), dtype=np.float64)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        y = (x[r0:r1].astype(np.float64) * s[None, :]).reshape(r1 - r0, p, m)
        nr = r1 - r0
        # over b': t[r, a', b] = sum_b' y[r, a', b'] * Hm[b, b']
        t = y @ hm.T
        # over a': z[r, a, b] = sum_a' H2[a, a'] * t[r, a', b], evaluated as
        # one matrix product with (r, b) as the batch of columns
        tt = np.ascontiguousarray(t.transpose(0, 2, 1)).reshape(nr * m, p)
        z = (tt @ h2.T).reshape(nr, m, p).transpose(0, 2, 1)
        out[r0:r1] = z.reshape(nr, d) * inv
    return out
