"""Pins for the oracle's Hadamard matrices (CPU only).

Each check ties the oracle to something outside its own code: a library
routine (scipy's Sylvester Hadamard), the recursion printed on the "QuaRot
Guide" page, properties the QuaRot paper-viz explainer states (two rows agree
in exactly half their positions; a one-hot vector maps to +-1/sqrt(d)), exact
integer orthogonality, and textbook identities of the Jacobsthal matrix and of
finite fields (which a wrong field table or a reducible modulus breaks).
"""

import itertools

import numpy as np
import pytest
import scipy.linalg

from oracle import GF, hadamard_m, paley1, sylvester
from oracle import hadamard as had_mod


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 64, 256, 1024, 4096])
def test_sylvester_matches_scipy(d):
    np.testing.assert_array_equal(sylvester(d), scipy.linalg.hadamard(d))


def test_sylvester_matches_doubling_recursion():
    # H_1 = [1]; H_2k = [[H_k, H_k], [H_k, -H_k]]
    h = np.ones((1, 1), dtype=np.int64)
    for _ in range(9):
        h = np.block([[h, h], [h, -h]])
        np.testing.assert_array_equal(sylvester(h.shape[0]), h)


@pytest.mark.parametrize("d", [2, 128, 4096])
def test_sylvester_exact_orthogonality(d):
    # float64 products of +-1 entries summed over d <= 4096 terms are exact
    h = sylvester(d).astype(np.float64)
    np.testing.assert_array_equal(h @ h.T, d * np.eye(d))


def test_rows_agree_in_half_the_positions():
    h = sylvester(256).astype(np.int64)
    agree = (h[:, None, :] == h[None, :, :]).sum(-1)
    off = agree[~np.eye(256, dtype=bool)]
    assert np.all(off == 128)


def test_one_hot_spreads_evenly():
    d = 4096
    h = sylvester(d).astype(np.float64) / np.sqrt(d)
    e = np.zeros(d)
    e[1234] = 1.0
    y = h @ e
    np.testing.assert_allclose(np.abs(y), 1.0 / np.sqrt(d), rtol=0, atol=1e-15)
    assert np.isclose(np.linalg.norm(y), 1.0, rtol=1e-14)


@pytest.mark.parametrize("m", [4, 8, 12, 20, 24, 28, 32])
def test_paley_is_hadamard_and_skew(m):
    h = hadamard_m(m).astype(np.int64)
    assert set(np.unique(h)) == {-1, 1}
    np.testing.assert_array_equal(h @ h.T, m * np.eye(m, dtype=np.int64))
    # skew-Hadamard: H + H^T = 2I
    np.testing.assert_array_equal(h + h.T, 2 * np.eye(m, dtype=np.int64))
    # normalised border of Paley I: first row all +1, first column -1 below it
    assert np.all(h[0] == 1)
    assert np.all(h[1:, 0] == -1)


@pytest.mark.parametrize("q", [3, 7, 11, 19, 23, 27, 31])
def test_jacobsthal_identities(q):
    h = paley1(q).astype(np.int64)
    jac = h[1:, 1:] - np.eye(q, dtype=np.int64)
    ones = np.ones((q, q), dtype=np.int64)
    np.testing.assert_array_equal(jac @ jac.T, q * np.eye(q, dtype=np.int64) - ones)
    np.testing.assert_array_equal(jac @ np.ones(q, dtype=np.int64), np.zeros(q, dtype=np.int64))
    np.testing.assert_array_equal(jac.T, -jac)  # q = 3 mod 4: chi(-1) = -1


def test_gf11_character_is_legendre_symbol():
    f = GF(11)
    for a in range(1, 11):
        euler = pow(a, 5, 11)  # Euler's criterion: a^((p-1)/2) = +-1 mod p
        assert f.chi(a) == (1 if euler == 1 else -1)


def test_gf27_field_axioms():
    f = GF(3, 3, modulus_low=(2, 2, 0))
    t = f.index([0, 1, 0])
    assert f.mul(f.mul(t, t), t) == f.add(t, f.index([1, 0, 0]))  # t^3 = t + 1
    one = f.index([1, 0, 0])
    for a in range(1, 27):
        assert sum(f.mul(a, b) == one for b in range(1, 27)) == 1
    for a, b, c in itertools.product(range(27), repeat=3):
        assert f.mul(f.mul(a, b), c) == f.mul(a, f.mul(b, c))
        assert f.mul(a, f.add(b, c)) == f.add(f.mul(a, b), f.mul(a, c))
    assert len(f.squares) == 13


def test_planted_reducible_modulus_is_caught(monkeypatch):
    # A wrong field table (t^3 + 1, which has the root t = 2 over GF(3)) must
    # fail the Hadamard pin.
    monkeypatch.setattr(had_mod, "_field_for", lambda q: GF(3, 3, modulus_low=(1, 0, 0)))
    h = had_mod.paley1(27).astype(np.int64)
    assert not np.array_equal(h @ h.T, 28 * np.eye(28, dtype=np.int64))


@pytest.mark.parametrize("a,b", [(2, 64), (16, 128), (32, 32), (256, 16)])
def test_sylvester_factors_as_kronecker_product(a, b):
    # (-1)^popcount(i & j) splits over the high and low index bits, so the
    # Sylvester matrix of order a b is H_a (x) H_b in natural order (the GPU
    # tests of large power-of-two rows take the oracle's rotation in this form)
    np.testing.assert_array_equal(np.kron(sylvester(a), sylvester(b)), sylvester(a * b))


def test_power_of_two_rotation_equals_its_kronecker_form():
    from oracle import rotate_rows

    rng = np.random.default_rng(3)
    d = 4096
    x = rng.standard_normal((5, d))
    s = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    np.testing.assert_allclose(rotate_rows(x, s, 128, hm=sylvester(128)), rotate_rows(x, s, 1),
                               rtol=0, atol=1e-12)
