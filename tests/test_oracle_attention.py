"""Pins of the oracle's decode attention over the INT4 cache.

The oracle follows "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs"
(paper-graph-ui summary), section 3.4: Stage 1d (the query is rotated
head-wise like the cached keys; softmax(q k^T / sqrt(d_h))), Stage 2c (the
decode-time list: dequantise each cached group on the fly) and Stage 1c
(the cross-head transform Z (H_{n_h} (x) I_{d_h})).  Pinned against
hand-derived cases (tests/golden/decode_example.json), the textbook
attention in the unrotated basis with scipy's softmax, the Kronecker
identity (I (x) H_{d_h})(H_{n_h} (x) I_{d_h}) = H_{n_h d_h}, and limiting
cases (one position, identical keys, a hard max, grouped heads = repeated
heads, lengths = truncation).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle.attention import attend, cross_head, decode_attention, dequant_cache, rotate_heads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "decode_example.json")


def random_cache(rng, b, h_kv, s, d, mode=0):
    """Random packed codes and fp16 scales (and zeros) of a [b, h_kv, s, d] cache."""
    if mode == 0:
        codes = rng.integers(-8, 8, size=(b, h_kv, s, d))
        k_q = oracle.pack_int4(codes)
        v_q = oracle.pack_int4(rng.integers(-8, 8, size=(b, h_kv, s, d)))
        cache = {"k_q": k_q, "v_q": v_q}
    else:
        cache = {"k_q": oracle.pack_uint4(rng.integers(0, 16, size=(b, h_kv, s, d))),
                 "v_q": oracle.pack_uint4(rng.integers(0, 16, size=(b, h_kv, s, d))),
                 "k_zero": rng.integers(-20, 21, size=(b, h_kv, s)).astype(np.float16),
                 "v_zero": rng.integers(-20, 21, size=(b, h_kv, s)).astype(np.float16)}
    cache["k_scale"] = rng.uniform(0.05, 0.5, size=(b, h_kv, s)).astype(np.float16)
    cache["v_scale"] = rng.uniform(0.05, 0.5, size=(b, h_kv, s)).astype(np.float16)
    return cache


def test_dequant_hand_derived():
    g = json.load(open(GOLDEN))["dequant"]
    sym = g["symmetric"]
    got = dequant_cache(np.array([sym["bytes"]], np.uint8), np.array([sym["scale"]], np.float16))
    assert got[0].tolist() == sym["values"], sym["derivation"]
    asy = g["asymmetric"]
    got = dequant_cache(np.array([asy["bytes"]], np.uint8), np.array([asy["scale"]], np.float16),
                        np.array([asy["zero"]], np.float16), mode=1)
    assert got[0].tolist() == asy["values"], asy["derivation"]


@pytest.mark.parametrize("idx", range(4))
def test_decode_hand_derived(idx):
    case = json.load(open(GOLDEN))["cases"][idx]
    b, hk, s = case["B"], case["H_kv"], case["S"]
    shape = (b, hk, s)
    cache = {"k_q": np.array(case["k_q"], np.uint8).reshape(*shape, 1),
             "v_q": np.array(case["v_q"], np.uint8).reshape(*shape, 1),
             "k_scale": np.array(case["k_scale"], np.float16).reshape(shape),
             "v_scale": np.array(case["v_scale"], np.float16).reshape(shape)}
    if case["mode"] == 1:
        cache["k_zero"] = np.array(case["k_zero"], np.float16).reshape(shape)
        cache["v_zero"] = np.array(case["v_zero"], np.float16).reshape(shape)
    q = np.array(case["q"], np.float16)
    out = decode_attention(q, np.array([1, 1], np.int8), cache, case["lengths"],
                           sm_scale=math.log(2.0) / math.sqrt(2.0), mode=case["mode"],
                           cross=case["cross"])
    np.testing.assert_allclose(out, np.array(case["out"]), rtol=0, atol=1e-14,
                               err_msg=case["derivation"])


@pytest.mark.parametrize("mode", [0, 1])
def test_equals_textbook_attention_in_unrotated_basis(mode):
    """R q against R k, R v gives R (attention of q, k, v): undo R on the cache,
    run textbook attention with scipy's softmax, rotate the result."""
    rng = np.random.default_rng(11)
    b, hk, hq, s, d = 2, 2, 4, 9, 16
    cache = random_cache(rng, b, hk, s, d, mode)
    signs = np.stack([(1 - 2 * rng.integers(0, 2, size=d)).astype(np.int8) for _ in range(hk)])
    q = rng.standard_normal((b, hq, d)).astype(np.float16)
    lengths = [9, 5]
    sm = 0.3
    got = decode_attention(q, signs, cache, lengths, sm_scale=sm, mode=mode)
    k_hat = dequant_cache(cache["k_q"], cache["k_scale"], cache.get("k_zero"), mode)
    v_hat = dequant_cache(cache["v_q"], cache["v_scale"], cache.get("v_zero"), mode)
    for bi in range(b):
        n = lengths[bi]
        for j in range(hq):
            kv = j // (hq // hk)
            r = oracle.dense_rotation(d, signs[kv])
            k_true = k_hat[bi, kv, :n] @ r  # rows: k^ = R k  ->  k = R^T k^
            v_true = v_hat[bi, kv, :n] @ r
            p = softmax(k_true @ q[bi, j].astype(np.float64) * sm)
            want = r @ (p @ v_true)
            np.testing.assert_allclose(got[bi, j], want, rtol=0, atol=1e-12)


def test_single_position_returns_its_value():
    rng = np.random.default_rng(2)
    cache = random_cache(rng, 2, 2, 5, 8)
    q = rng.standard_normal((2, 4, 8)).astype(np.float16)
    out = decode_attention(q, np.ones(8, np.int8), cache, [1, 1])
    v_hat = dequant_cache(cache["v_q"], cache["v_scale"])
    for j in range(4):
        np.testing.assert_allclose(out[:, j], v_hat[:, j // 2, 0], rtol=0, atol=1e-15)


def test_identical_keys_average_the_values():
    rng = np.random.default_rng(3)
    cache = random_cache(rng, 1, 1, 7, 16)
    cache["k_q"][:] = cache["k_q"][:, :, :1]
    cache["k_scale"][:] = cache["k_scale"][:, :, :1]
    q = rng.standard_normal((1, 1, 16)).astype(np.float16)
    out = decode_attention(q, np.ones(16, np.int8), cache, [6])
    v_hat = dequant_cache(cache["v_q"], cache["v_scale"])
    np.testing.assert_allclose(out[0, 0], v_hat[0, 0, :6].mean(axis=0), rtol=0, atol=1e-14)


def test_large_scale_selects_the_best_key():
    """With a huge softmax scale the output is the value of the top-scoring key
    (a sign error in the scores would pick the lowest one)."""
    rng = np.random.default_rng(4)
    d = 32
    cache = random_cache(rng, 1, 1, 12, d)
    signs = (1 - 2 * rng.integers(0, 2, size=d)).astype(np.int8)
    q = rng.standard_normal((1, 1, d)).astype(np.float16)
    k_hat = dequant_cache(cache["k_q"], cache["k_scale"])
    scores = k_hat[0, 0] @ rotate_heads(q, signs, 1)[0, 0]
    order = np.argsort(scores)
    assert scores[order[-1]] - scores[order[-2]] > 1e-3
    out = decode_attention(q, signs, cache, [12], sm_scale=1e6)
    v_hat = dequant_cache(cache["v_q"], cache["v_scale"])
    np.testing.assert_allclose(out[0, 0], v_hat[0, 0, order[-1]], rtol=0, atol=1e-12)


def test_grouped_heads_equal_repeated_heads():
    """H_kv = 2, H_q = 8 gives the same result as 8 KV heads where head j is a
    copy of KV head j // 4 (consecutive query heads share a KV head)."""
    rng = np.random.default_rng(5)
    d = 16
    cache = random_cache(rng, 2, 2, 6, d, mode=1)
    signs = np.stack([(1 - 2 * rng.integers(0, 2, size=d)).astype(np.int8) for _ in range(2)])
    q = rng.standard_normal((2, 8, d)).astype(np.float16)
    got = decode_attention(q, signs, cache, [6, 4], mode=1)
    rep = {k: np.repeat(v, 4, axis=1) for k, v in cache.items()}
    want = decode_attention(q, np.repeat(signs, 4, axis=0), rep, [6, 4], mode=1)
    np.testing.assert_array_equal(got, want)
    # and a different grouping (head j -> j % 2) does not give it
    alt = {k: np.tile(v, (1, 4) + (1,) * (v.ndim - 2)) for k, v in cache.items()}
    other = decode_attention(q, np.tile(signs, (4, 1)), alt, [6, 4], mode=1)
    assert np.abs(other - want).max() > 1e-3


def test_lengths_equal_truncation_and_ignore_the_tail():
    rng = np.random.default_rng(6)
    cache = random_cache(rng, 1, 2, 10, 8)
    q = rng.standard_normal((1, 2, 8)).astype(np.float16)
    got = decode_attention(q, np.ones(8, np.int8), cache, [7])
    cut = {k: v[:, :, :7] for k, v in cache.items()}
    np.testing.assert_array_equal(got, decode_attention(q, np.ones(8, np.int8), cut, [7]))
    cache["k_q"][:, :, 7:] = 0x77
    cache["v_q"][:, :, 7:] = 0x77
    np.testing.assert_array_equal(got, decode_attention(q, np.ones(8, np.int8), cache, [7]))


def test_zero_length_row_is_zero():
    rng = np.random.default_rng(7)
    cache = random_cache(rng, 2, 1, 4, 8)
    q = rng.standard_normal((2, 1, 8)).astype(np.float16)
    out = decode_attention(q, np.ones(8, np.int8), cache, [0, 4])
    assert not out[0].any()
    assert np.abs(out[1]).max() > 0


def test_cross_head_completes_the_full_hadamard():
    """(I_{n_h} (x) H_{d_h}) then (H_{n_h} (x) I_{d_h}) is H_{n_h d_h} (Sylvester,
    normalised): per-head transform + cross_head = dense transform of the row."""
    rng = np.random.default_rng(8)
    nh, dh = 4, 8
    z = rng.standard_normal((3, nh, dh))
    per_head = np.einsum("bhd,ed->bhe", z, oracle.sylvester(dh).astype(np.float64)) / math.sqrt(dh)
    got = cross_head(per_head).reshape(3, nh * dh)
    want = z.reshape(3, nh * dh) @ oracle.sylvester(nh * dh).astype(np.float64).T / math.sqrt(nh * dh)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_cross_head_is_an_involution_and_keeps_the_norm():
    rng = np.random.default_rng(9)
    z = rng.standard_normal((2, 16, 5))
    np.testing.assert_allclose(cross_head(cross_head(z)), z, rtol=0, atol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(cross_head(z)), np.linalg.norm(z), rtol=1e-14)


def test_attend_softmax_shift_invariance():
    """Adding a constant to every score (a key component along q) changes nothing:
    the softmax normalises it away (checks the max-subtraction bookkeeping)."""
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 1, 4))
    k = rng.standard_normal((1, 1, 6, 4))
    v = rng.standard_normal((1, 1, 6, 4))
    base = attend(q, k, v, [6], 0.7)
    shifted = attend(q, k + 40.0 * q[:, :, None, :] / np.dot(q[0, 0], q[0, 0]), v, [6], 0.7)
    np.testing.assert_allclose(shifted, base, rtol=0, atol=1e-12)
