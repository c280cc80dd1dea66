"""Pins of the oracle's gated-product rotate+quant (``oracle.swiglu_had_quant``).

"QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
summary), section 3.4 "FFN Activation Rotation (Stage 1b)": the
down-projection input is c = SiLU(A) * B and the online Hadamard acts on c.
SiLU is pinned against scipy's logistic function, closed forms and
hand-evaluated values; the fused step against the plain rotate+quant of an
independently formed product and a one-hot case whose rotation is exact.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_silu_matches_scipy_logistic():
    t = np.linspace(-40.0, 40.0, 4001)
    np.testing.assert_allclose(oracle.silu(t), t * expit(t), rtol=1e-14, atol=1e-300)


def test_silu_closed_forms():
    t = np.linspace(-20.0, 20.0, 801)
    # sigmoid(-t) = 1 - sigmoid(t)  =>  SiLU(t) - SiLU(-t) = t
    np.testing.assert_allclose(oracle.silu(t) - oracle.silu(-t), t, rtol=0, atol=1e-13)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    # far tails: t itself, and a vanishing negative value (no overflow to nan)
    big = oracle.silu(np.array([60.0, -1000.0]))
    assert big[0] == 60.0 and big[1] == 0.0 and np.all(np.isfinite(big))


def test_hand_evaluated_products():
    with open(os.path.join(GOLDEN, "swiglu_example.json")) as f:
        g = json.load(f)
    np.testing.assert_allclose(oracle.silu(np.array(g["gate"])), g["silu_gate"], rtol=1e-15)
    np.testing.assert_allclose(oracle.swiglu(np.array(g["gate"]), np.array(g["up"])),
                               g["product"], rtol=1e-15)
    # SiLU(1) = e / (e + 1), the page's sigmoid form
    assert math.isclose(g["silu_gate"][0], math.e / (math.e + 1.0), rel_tol=1e-15)


def test_one_hot_product_spreads_to_the_hadamard_column():
    with open(os.path.join(GOLDEN, "swiglu_example.json")) as f:
        g = json.load(f)["one_hot"]
    d, k = g["d"], g["k"]
    rng = np.random.default_rng(0)
    gate = rng.standard_normal((1, d))
    up = np.zeros((1, d))
    gate[0, k], up[0, k] = g["gate_k"], g["up_k"]
    s = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    r = oracle.swiglu_had_quant(gate, up, s)
    np.testing.assert_allclose(np.abs(r["x_rot"][0]), g["abs_rotated"], rtol=1e-14)
    want_sign = s[k] * oracle.sylvester(d)[:, k]
    np.testing.assert_array_equal(np.sign(r["x_rot"][0]), want_sign)
    np.testing.assert_array_equal(r["codes"][0], 7 * want_sign)
    assert r["scales"][0] == np.float16(g["c"] / math.sqrt(d) / 7.0)


@pytest.mark.parametrize("d,m", [(256, 1), (4096, 1), (1536, 12), (3584, 28)])
def test_fused_step_equals_rotate_quant_of_the_product(d, m):
    rng = np.random.default_rng(d + m)
    gate = rng.standard_normal((9, d)).astype(np.float16)
    up = rng.standard_normal((9, d)).astype(np.float16)
    s = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    prod = gate.astype(np.float64) * expit(gate.astype(np.float64)) * up.astype(np.float64)
    want = oracle.had_quant(prod, s, m)
    got = oracle.swiglu_had_quant(gate, up, s, m)
    np.testing.assert_allclose(got["x_rot"], want["x_rot"], rtol=0,
                               atol=1e-13 * np.abs(want["x_rot"]).max())
    np.testing.assert_array_equal(got["scales"], want["scales"])
    np.testing.assert_array_equal(got["codes"], want["codes"])


def test_planted_gate_up_swap_is_caught():
    # SiLU applies to the gate only: swapping the operands changes the product
    rng = np.random.default_rng(2)
    a, b = rng.standard_normal((2, 3, 64))
    assert np.abs(oracle.swiglu(a, b) - oracle.swiglu(b, a)).max() > 1e-2
