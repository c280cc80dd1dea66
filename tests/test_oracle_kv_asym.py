"""Pins of the oracle's asymmetric (zero-point) group quantiser.

The quantiser follows the Stage 2c description of "QuaRot: Outlier-Free
4-Bit Inference in Rotated LLMs" (paper-graph-ui summary, section 3.4):
scale = clipped range / 15, integer zero point, uint4 codes.  Pinned against
hand-derived values (tests/golden/asym_example.json), a brute-force nearest
grid point search, reconstruction bounds and symmetry properties.
"""

from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "asym_example.json")


def test_asym_hand_derived_cases():
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        x = np.array([case["x"]], dtype=np.float64)
        codes, s, z = oracle.quantize_rows_asym(x, case["clip"])
        want_s = case["scale"] if "scale" in case else float(np.float16(case["scale_fp16_of"]))
        assert float(s[0]) == want_s, case["derivation"]
        assert int(z[0]) == case["zero"], case["derivation"]
        assert codes[0].tolist() == case["codes"], case["derivation"]


def test_uint4_packing_golden_and_roundtrip():
    g = json.load(open(GOLDEN))["packing"]
    packed = oracle.pack_uint4(np.array([g["codes"]]))
    assert packed[0].tolist() == g["bytes"]
    rng = np.random.default_rng(4)
    q = rng.integers(0, 16, size=(7, 64)).astype(np.uint8)
    np.testing.assert_array_equal(oracle.unpack_uint4(oracle.pack_uint4(q)), q)
    with pytest.raises(ValueError):
        oracle.pack_uint4(np.array([[16, 0]]))


@pytest.mark.parametrize("clip", [1.0, 0.95])
def test_asym_codes_are_nearest_grid_points(clip):
    # brute force over the 16 levels S * (q - z): the code is the nearest one
    # (clamped values excepted when clip < 1)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((200, 32)) * rng.uniform(0.01, 50, (200, 1)) + rng.normal(0, 3, (200, 1))
    codes, s, z = oracle.quantize_rows_asym(x, clip)
    s64 = s.astype(np.float64)[:, None]
    levels = s64[:, :, None] * (np.arange(16)[None, None, :] - z[:, None, None])
    dist = np.abs(x[:, :, None] - levels)
    best = dist.min(axis=2)
    got = np.take_along_axis(dist, codes[:, :, None].astype(np.int64), axis=2)[:, :, 0]
    # the decision is the float64 definition: nearest level up to round-off
    assert np.all(got <= best + 1e-12 * s64)


def test_asym_reconstruction_bound_and_range():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((300, 128)) + rng.normal(0, 2, (300, 1))
    codes, s, z = oracle.quantize_rows_asym(x, 1.0)
    assert codes.min() >= 0 and codes.max() <= 15
    xhat = s.astype(np.float64)[:, None] * (codes.astype(np.float64) - z[:, None])
    err = np.abs(xhat - x)
    s64 = s.astype(np.float64)[:, None]
    # half a step, plus the fp16 rounding of the scale across 15 steps
    assert np.all(err <= s64 * (0.5 + 16 * 2.0 ** -10) + 1e-12)
    # clip 1: the group extremes land on (or next to) codes 0 and 15
    assert np.all(codes.min(axis=1) <= 1) and np.all(codes.max(axis=1) >= 14)


def test_asym_symmetric_group_zero_point():
    # a group symmetric about 0 has -alpha_min / S = 7.5 up to the fp16 scale
    rng = np.random.default_rng(7)
    h = np.abs(rng.standard_normal((50, 16))) + 0.1
    x = np.concatenate([h, -h], axis=1)
    _, _, z = oracle.quantize_rows_asym(x, 0.95)
    assert set(np.unique(z)) <= {7, 8}


def test_asym_planted_sign_error_is_caught():
    # the zero point taken as rint(+alpha_min / S) (the page's garbled sign)
    # must disagree with the hand-derived case
    x = np.array([[-1.0, 0.0, 0.5, 2.0]])
    s, z = oracle.asym_params(x, 1.0)
    wrong = np.clip(np.rint(-1.0 / s.astype(np.float64)), -oracle.ZMAX, oracle.ZMAX)
    assert int(wrong[0]) != int(z[0])


def test_kv_asym_uses_the_symmetric_rotation():
    cfg = workloads.KV_CONFIG
    inp = workloads.make_kv_inputs(cfg, batch=1, heads=2, positions=8)
    a = oracle.kv_had_quant_asym(inp["k"], inp["signs"])
    b = oracle.kv_had_quant(inp["k"], inp["signs"])
    np.testing.assert_array_equal(a["x_rot"], b["x_rot"])
    d = inp["k"].shape[-1]
    codes, s, z = oracle.quantize_rows_asym(a["x_rot"].reshape(-1, d), 0.95)
    np.testing.assert_array_equal(a["codes"].reshape(-1, d), codes)
    np.testing.assert_array_equal(oracle.unpack_uint4(a["packed"]).reshape(-1, d), codes)
