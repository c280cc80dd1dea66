"""Pins of the oracle's RMSNorm-fused rotate+quant.

Follows "QuaRot Guide: Outlier-Free 4-Bit W4A4 LLM Quantization", step 2 of
"Deep Dive" (the online rotation fused into RMSNorm: normalise, rotate,
quantise per token), with the gain absorbed into the next weights
("QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs", paper-graph-ui
summary, Stage 1a).  Pinned by hand-derived cases
(tests/golden/rmsnorm_example.json), the closed form of the mean square
after normalisation, scale invariance, and the norm the orthogonal rotation
must keep.
"""

from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rmsnorm_example.json")


@pytest.mark.parametrize("idx", range(2))
def test_rmsnorm_hand_derived(idx):
    case = json.load(open(GOLDEN))["cases"][idx]
    r = oracle.rmsnorm_had_quant(np.array([case["x"]]), np.array(case["signs"], np.int8), 1, 1.0,
                                 case["eps"])
    np.testing.assert_allclose(r["x_rot"][0], case["x_rot"], rtol=0, atol=1e-14,
                               err_msg=case["derivation"])
    assert float(r["scales"][0]) == case["scale"], case["derivation"]
    assert r["codes"][0].tolist() == case["codes"], case["derivation"]


def test_mean_square_closed_form():
    """mean(y^2) = ms / (ms + eps) with ms = mean(x^2): 1 at eps = 0."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64)) * np.array([[0.01], [0.1], [1.0], [10.0], [100.0]])
    for eps in (0.0, 1e-6, 1e-2):
        y = oracle.rmsnorm(x, eps)
        ms = np.mean(x * x, axis=1)
        np.testing.assert_allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-13, atol=0)


def test_scale_invariance_at_zero_eps():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 128))
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * x, 0.0), oracle.rmsnorm(x, 0.0), rtol=1e-14,
                               atol=0)


@pytest.mark.parametrize("d,m", [(256, 1), (384, 12), (896, 28)])
def test_rotated_rows_keep_the_normalised_norm(d, m):
    """||R y||^2 = d * ms / (ms + eps): the rotation is orthogonal and the
    normalisation divides by the root of the *mean* square."""
    rng = np.random.default_rng(d)
    x = (rng.standard_normal((4, d)) * 3.0).astype(np.float16)
    signs = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    eps = 1e-3
    r = oracle.rmsnorm_had_quant(x, signs, m, 1.0, eps)
    x64 = x.astype(np.float64)
    ms = np.mean(x64 * x64, axis=1)
    np.testing.assert_allclose(np.sum(r["x_rot"] ** 2, axis=1), d * ms / (ms + eps), rtol=1e-12)


def test_equals_scaled_plain_rotation():
    """Rotating the normalised row equals scaling the rotated raw row by the
    per-row factor; the codes then match the plain path's up to ties."""
    rng = np.random.default_rng(3)
    d = 512
    x = (rng.standard_normal((32, d)) * 2.0).astype(np.float16)
    signs = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    eps = 1e-5
    fused = oracle.rmsnorm_had_quant(x, signs, 1, 1.0, eps)
    plain = oracle.had_quant(x, signs, 1)
    x64 = x.astype(np.float64)
    rr = 1.0 / np.sqrt(np.mean(x64 * x64, axis=1, keepdims=True) + eps)
    np.testing.assert_allclose(fused["x_rot"], plain["x_rot"] * rr, rtol=1e-12, atol=1e-15)
    assert np.mean(fused["codes"] != plain["codes"]) < 5e-3
