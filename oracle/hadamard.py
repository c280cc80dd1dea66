"""Hadamard matrices for the oracle: Sylvester H_{2^n} and Paley-I H_m.

Sources (page titles; no other file is cited):

* "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
  summary), section 3.4, "Computational Invariance and Between-Block Rotation
  (Stage 1a)": the randomized Hadamard is H * diag(s); when d is not a power of
  two it is factored as d = 2^n * m with H_d = H_{2^n} (x) H_m, H_m a known
  Hadamard matrix of size m.
* "QuaRot Guide: Outlier-Free 4-Bit W4A4 LLM Quantization" (aifetchly blog),
  section "2. Why Randomized Walsh-Hadamard Transforms (RHT) Disperse
  Outliers": the Sylvester recursion H_{2k} = [[H_k, H_k], [H_k, -H_k]].
* QuaRot paper-viz explainer (romaanj.github.io), the table of how the matrix
  is built at each size: Sylvester for 2^n, and a Kronecker product with a
  Paley block of size 12 for width 12288.

The pages never print H_12 or H_28.  Any Hadamard matrix of that order is a
valid choice; this module fixes the classical Paley construction of type I
(order q + 1 for a prime power q = 3 mod 4) with the element orderings stated
below.  The HIP library carries its own, independently written construction
of the same matrices; the two agree only if both follow the same definition.

Everything here is exact integer arithmetic (numpy int64), returned as int8.
"""

from __future__ import annotations

import functools
import itertools

import numpy as np

__all__ = [
    "sylvester",
    "GF",
    "paley1",
    "hadamard_m",
    "SUPPORTED_M",
]


def sylvester(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d = 2^n, entries +-1 (int8).

    Closed form of the doubling recursion: entry (i, j) is (-1) raised to the
    number of bit positions where both i and j have a 1.
    """
    if d < 1 or (d & (d - 1)) != 0:
        raise ValueError(f"Sylvester order must be a power of two, got {d}")
    i = np.arange(d, dtype=np.int64)
    both = i[:, None] & i[None, :]
    # popcount parity, bit by bit (d <= 2^16 here)
    parity = np.zeros_like(both)
    bits = both.copy()
    while np.any(bits):
        parity ^= bits & 1
        bits >>= 1
    return (1 - 2 * parity).astype(np.int8)


class GF:
    """The finite field GF(q) for q = p (prime) or q = p^k, elements indexed 0..q-1.

    Element with index i is the polynomial sum_k c_k t^k over GF(p), where
    c_k is the k-th base-p digit of i (c_0 least significant).  For prime q
    this is just the integer i mod p.  Multiplication reduces modulo the given
    monic irreducible polynomial (coefficients low to high, leading 1 implied).
    """

    def __init__(self, p: int, k: int = 1, modulus_low=()):
        self.p = p
        self.k = k
        self.q = p ** k
        if k > 1 and len(modulus_low) != k:
            raise ValueError("need k low-order coefficients of the modulus")
        self.modulus_low = tuple(int(c) % p for c in modulus_low)

    def digits(self, i: int):
        out = []
        for _ in range(self.k):
            out.append(i % self.p)
            i //= self.p
        return out

    def index(self, coeffs) -> int:
        i = 0
        for c in reversed(coeffs):
            i = i * self.p + (c % self.p)
        return i

    def add(self, a: int, b: int) -> int:
        da, db = self.digits(a), self.digits(b)
        return self.index([x + y for x, y in zip(da, db)])

    def neg(self, a: int) -> int:
        return self.index([-x for x in self.digits(a)])

    def sub(self, a: int, b: int) -> int:
        return self.add(a, self.neg(b))

    def mul(self, a: int, b: int) -> int:
        p, k = self.p, self.k
        da, db = self.digits(a), self.digits(b)
        prod = [0] * (2 * k - 1)
        for i, x in enumerate(da):
            for j, y in enumerate(db):
                prod[i + j] = (prod[i + j] + x * y) % p
        # reduce: t^k = -(modulus_low . (1, t, ..., t^{k-1}))
        for deg in range(2 * k - 2, k - 1, -1):
            c = prod[deg]
            if c:
                prod[deg] = 0
                for j, mcoef in enumerate(self.modulus_low):
                    prod[deg - k + j] = (prod[deg - k + j] - c * mcoef) % p
        return self.index(prod[:k])

    @functools.cached_property
    def squares(self) -> frozenset:
        return frozenset(self.mul(x, x) for x in range(1, self.q))

    def chi(self, a: int) -> int:
        """Quadratic character: 0 at 0, +1 on nonzero squares, -1 otherwise."""
        if a == 0:
            return 0
        return 1 if a in self.squares else -1


def _field_for(q: int) -> GF:
    if q == 27:
        # GF(27) = GF(3)[t] / (t^3 + 2t + 2); the cubic has no root mod 3.
        return GF(3, 3, modulus_low=(2, 2, 0))
    for p in range(2, q):
        if q % p == 0:
            raise ValueError(f"no field table for q = {q}")
    return GF(q)


def paley1(q: int) -> np.ndarray:
    """Paley construction I: Hadamard matrix of order m = q + 1 (int8).

    Requires q = 3 (mod 4).  With the field elements in index order,
      Jacobsthal  Q[i, j] = chi(e_i - e_j)            (q x q)
      S = [[0, 1^T], [-1, Q]]                         (m x m, skew)
      H = I + S.
    """
    if q % 4 != 3:
        raise ValueError("Paley I needs q = 3 mod 4")
    f = _field_for(q)
    jac = np.zeros((q, q), dtype=np.int64)
    for i, j in itertools.product(range(q), range(q)):
        jac[i, j] = f.chi(f.sub(i, j))
    m = q + 1
    s = np.zeros((m, m), dtype=np.int64)
    s[0, 1:] = 1
    s[1:, 0] = -1
    s[1:, 1:] = jac
    h = np.eye(m, dtype=np.int64) + s
    return h.astype(np.int8)


# Orders with a Paley type-I matrix here: q = m - 1 a prime (or 27) with
# q = 3 mod 4.  (16 has none: 15 is not a prime power.)
SUPPORTED_M = (1, 4, 8, 12, 20, 24, 28, 32)


@functools.lru_cache(maxsize=None)
def _hadamard_m_cached(m: int) -> bytes:
    if m == 1:
        h = np.ones((1, 1), dtype=np.int8)
    elif m in SUPPORTED_M:
        h = paley1(m - 1)
    else:
        raise ValueError(f"no small Hadamard factor of order {m} (have {SUPPORTED_M})")
    return h.tobytes()


def hadamard_m(m: int) -> np.ndarray:
    """The small Kronecker factor H_m used for d = 2^n * m (int8 [m x m]):
    [1] for m = 1, else the Paley type-I matrix of order m."""
    return np.frombuffer(_hadamard_m_cached(m), dtype=np.int8).reshape(m, m).copy()
