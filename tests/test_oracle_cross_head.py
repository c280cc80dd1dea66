"""Pins of the oracle's cross-head transform + per-token quantisation.

Follows "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
summary), section 3.4 Stage 1c: the attention output Z (heads concatenated)
gets Z (H_{n_h} (x) I_{d_h}) online before the out-projection, and the full
Hadamard factors as H_{n_h d_h} = (I_{n_h} (x) H_{d_h}) (H_{n_h} (x) I_{d_h});
then Stage 2b's per-token quantiser.  Pinned by hand-derived cases
(tests/golden/cross_head_example.json), that factorisation against the
independently pinned full-width rotation, brute force on a tiny input with a
Hadamard built by the block recursion, the involution and norm of the
normalised transform, and the quantiser's error bound.
"""

from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cross_head_example.json")


@pytest.mark.parametrize("idx", range(2))
def test_cross_head_hand_derived(idx):
    case = json.load(open(GOLDEN))["cases"][idx]
    r = oracle.cross_head_quant(np.array([case["z"]]), case["n_heads"])
    np.testing.assert_allclose(r["x_rot"][0], case["z_rot"], rtol=0, atol=1e-14,
                               err_msg=case["derivation"])
    assert float(r["scales"][0]) == case["scale"], case["derivation"]
    assert r["codes"][0].tolist() == case["codes"], case["derivation"]


@pytest.mark.parametrize("nh,dh", [(2, 8), (8, 16), (32, 128)])
def test_factorisation_of_the_full_hadamard(nh, dh):
    """Head-wise H_{d_h} on each head, then the cross-head transform, equals
    the full-width Sylvester rotation (all signs +1) of the row."""
    rng = np.random.default_rng(nh * dh)
    z = rng.standard_normal((5, nh * dh))
    ones_h = np.ones(dh, dtype=np.int8)
    per_head = oracle.rotate_rows(z.reshape(-1, dh), ones_h, 1).reshape(5, nh * dh)
    got = oracle.cross_head_quant(per_head, nh)["x_rot"]
    want = oracle.rotate_rows(z, np.ones(nh * dh, dtype=np.int8), 1)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def _block_recursion(n: int) -> np.ndarray:
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_brute_force_tiny():
    """z~[t, a*d_h + c] = sum_a' H[a', a] z[t, a'*d_h + c] / sqrt(n_h), by loops."""
    nh, dh, t = 4, 3, 2
    rng = np.random.default_rng(7)
    z = rng.standard_normal((t, nh * dh))
    h = _block_recursion(nh)
    want = np.zeros_like(z)
    for r in range(t):
        for a in range(nh):
            for c in range(dh):
                want[r, a * dh + c] = sum(h[ap, a] * z[r, ap * dh + c] for ap in range(nh)) / 2.0
    np.testing.assert_allclose(oracle.cross_head_quant(z, nh)["x_rot"], want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("nh", [2, 16, 64])
def test_involution_and_norm(nh):
    rng = np.random.default_rng(nh)
    z = rng.standard_normal((3, nh * 128))
    once = oracle.cross_head_quant(z, nh)["x_rot"]
    twice = oracle.cross_head_quant(once, nh)["x_rot"]
    np.testing.assert_allclose(twice, z, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(once, axis=1), np.linalg.norm(z, axis=1), rtol=1e-13)


def test_quantiser_error_bound_and_extremes():
    cfg = workloads.CROSS_HEAD_CONFIGS["attn_out_7b"]
    z = workloads.make_attn_output(cfg, tokens=16)["z"]
    r = oracle.cross_head_quant(z, cfg.heads)
    s = r["scales"].astype(np.float64)[:, None]
    assert np.all(np.abs(r["codes"] * s - r["x_rot"]) <= s / 2 * (1 + 1e-12))
    # the row's largest magnitude lands on +-7 (S is max / 7 rounded to fp16)
    top = np.abs(r["codes"]).max(axis=1)
    assert np.all(top == 7)
    assert np.array_equal(oracle.unpack_int4(r["packed"]), r["codes"])


def test_loud_heads_are_spread():
    """With a few heads far louder than the rest, the transform gives every
    head the same share of the row's energy (each output head is a +-1 mix of
    all input heads), so per-head energies even out."""
    cfg = workloads.CROSS_HEAD_CONFIGS["attn_out_70b"]
    z = workloads.make_attn_output(cfg, tokens=8)["z"].astype(np.float64)
    r = oracle.cross_head_quant(z, cfg.heads)["x_rot"]
    before = (z.reshape(8, cfg.heads, -1) ** 2).sum(axis=2)
    after = (r.reshape(8, cfg.heads, -1) ** 2).sum(axis=2)
    assert np.all(before.max(axis=1) / before.mean(axis=1) > 10)
    assert np.all(after.max(axis=1) / after.mean(axis=1) < 1.5)


def test_rejects_bad_head_count():
    with pytest.raises(ValueError):
        oracle.cross_head_quant(np.zeros((1, 12)), 5)
