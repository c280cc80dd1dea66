"""Pins for the oracle's quantiser, packing, integer GEMM and dequant (CPU only).

Closed forms from "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs"
(paper-graph-ui summary, section 3.4 Stage 2a/2b: s = max/(2^(b-1) - 1),
round to nearest) and "QuaRot Guide" (clip to [-8, 7], S = max|X| / 7,
absmax floor 1e-5), worked fixtures under tests/golden/, and exact integer
arithmetic for the GEMM.
"""

import json
import os

import numpy as np
import pytest

import workloads
from oracle import (codes_from_scales, dequant, int_gemm, int_gemm_exact,
                    pack_int4, quantize_rows, rotate_rows, row_scales,
                    unpack_int4, w4a4_linear)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_scale_is_max_over_seven_in_fp16():
    x = np.array([[3.5, -7.0, 1.0, 0.0]])
    s = row_scales(x)
    assert s.dtype == np.float16 and float(s[0]) == 1.0
    s9 = row_scales(x, 0.9)
    assert float(s9[0]) == float(np.float16(0.9 * 7.0 / 7.0))


def test_multiples_of_the_scale_round_trip():
    s = np.float16(0.125)
    ks = np.arange(-7, 8)
    x = (ks * float(s)).reshape(1, -1)
    q, sc = quantize_rows(x)
    assert float(sc[0]) == float(s)  # max 0.875 -> 0.875/7 = 0.125 exactly
    np.testing.assert_array_equal(q[0], ks)


def test_ties_round_to_even():
    s = np.array([np.float16(0.25)])
    x = (np.arange(-7, 7) + 0.5).reshape(1, -1) * 0.25
    q = codes_from_scales(x, s)[0]
    want = np.array([-6, -6, -4, -4, -2, -2, 0, 0, 2, 2, 4, 4, 6, 6])
    np.testing.assert_array_equal(q, want)


def test_decision_is_taken_on_the_exact_value():
    # x / S a hair above or below k + 1/2: rint of the exact quotient (ties
    # to even only at an exact tie).  A decision taken on fp32-rounded values
    # would see 2.5 and 4.5 here and round both to even.
    s = np.array([np.float16(1.0)])
    x = np.array([[2.5 + 2.0 ** -40, 4.5 - 2.0 ** -40, -2.5 - 2.0 ** -40, 2.5]])
    assert np.float32(x[0, 0]) == np.float32(2.5)  # the fp32 view is a tie
    np.testing.assert_array_equal(codes_from_scales(x, s)[0], [3, 4, -3, 2])


def test_absmax_maps_to_seven():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, 333))
    q, _ = quantize_rows(x)
    amax = np.argmax(np.abs(x), axis=1)
    np.testing.assert_array_equal(np.abs(q[np.arange(50), amax]), 7)
    assert q.min() >= -7 and q.max() <= 7  # clip 1.0 never reaches -8


def test_clip_below_one_saturates():
    x = np.array([[-10.0, 10.0, 0.1]])
    q, s = quantize_rows(x, clip_ratio=0.5)
    assert float(s[0]) == float(np.float16(5.0 / 7.0))
    assert q[0, 0] == -8 and q[0, 1] == 7


def test_zero_row_uses_floor():
    q, s = quantize_rows(np.zeros((2, 16)))
    assert np.all(q == 0)
    assert float(s[0]) == float(np.float16(1e-5 / 7))


def test_page_outlier_example():
    with open(os.path.join(GOLDEN, "p3_outlier_row.json")) as f:
        g = json.load(f)
    q, s = quantize_rows(np.array([g["row"]]), g["clip_ratio"])
    assert float(s[0]) == g["scale_fp16"]
    np.testing.assert_array_equal(q[0], g["codes"])


def test_pack_examples():
    with open(os.path.join(GOLDEN, "pack_examples.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        b = pack_int4(np.array([c["codes"]]))
        assert int(b[0, 0]) == c["byte"], c
        np.testing.assert_array_equal(unpack_int4(b)[0], c["codes"])


def test_pack_round_trip():
    rng = np.random.default_rng(0)
    q = rng.integers(-8, 8, size=(9, 64)).astype(np.int8)
    np.testing.assert_array_equal(unpack_int4(pack_int4(q)), q)


def test_blas_gemm_is_exact():
    rng = np.random.default_rng(2)
    for k in (256, 4096, 28672):
        a = rng.integers(-8, 8, size=(17, k)).astype(np.int8)
        b = rng.integers(-8, 8, size=(13, k)).astype(np.int8)
        np.testing.assert_array_equal(int_gemm(a, b), int_gemm_exact(a, b))


def test_gemm_extreme_accumulator():
    k = 28672
    a = np.full((1, k), -8, np.int8)
    acc = int_gemm(a, a)
    assert int(acc[0, 0]) == 64 * k == 1835008
    assert acc[0, 0] < 2 ** 31


def test_dequant_closed_form():
    acc = np.array([[100, -3], [0, 70000]])
    sx = np.array([0.5, 2.0], np.float16)
    sw = np.array([0.25, 1.0], np.float16)
    y = dequant(acc, sx, sw)
    np.testing.assert_array_equal(
        y, np.array([[12.5, -1.5], [0.0, np.inf]], dtype=np.float16))


def test_rotation_reduces_w4a4_error():
    cfg = workloads.ACT_CONFIGS["tiny"]
    inp = workloads.make_act_inputs(cfg)
    x = inp["x"].astype(np.float64)
    w = inp["w"].astype(np.float64)
    ref = x @ w.T
    rot = w4a4_linear(inp["x"], inp["w"], inp["signs"])["y"].astype(np.float64)
    qx, sx = quantize_rows(x)
    qw, sw = quantize_rows(w)
    naive = dequant(int_gemm(qx, qw), sx, sw).astype(np.float64)
    e_rot = np.linalg.norm(rot - ref) / np.linalg.norm(ref)
    e_naive = np.linalg.norm(naive - ref) / np.linalg.norm(ref)
    assert e_rot < 0.7 * e_naive


def test_rotated_weights_have_flat_channel_scales():
    # After rotation every output channel's row is spread evenly, so
    # max/7 codes use the whole [-7, 7] range on every row.
    cfg = workloads.ACT_CONFIGS["tiny"]
    inp = workloads.make_act_inputs(cfg)
    wr = rotate_rows(inp["w"], inp["signs"])
    q, s = quantize_rows(wr)
    assert np.all(np.abs(q).max(axis=1) == 7)


def test_planted_dropped_scale_is_caught():
    # Dequant that forgets the weight scale must be far from the reference.
    cfg = workloads.ACT_CONFIGS["tiny"]
    inp = workloads.make_act_inputs(cfg)
    r = w4a4_linear(inp["x"], inp["w"], inp["signs"])
    bad = dequant(r["acc"], r["act"]["scales"], np.ones_like(r["wgt"]["scales"]))
    assert not np.allclose(bad.astype(float), r["y"].astype(float), rtol=1e-2)
