"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Every case prints its name and shape before touching the GPU.  Inputs come
from the seeded generators in ``workloads``; expected values only from
``oracle``.  Comparison rules are in ``parity.py``.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from parity import (check_asym, check_codes, check_quant, check_rot, check_y_elementwise,
                    check_y_frobenius)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotated_w4a4_amd as qr  # noqa: E402


def say(msg: str) -> None:
    print(f"[parity] {msg}", flush=True)


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_had_quant(x16: np.ndarray, signs, m: int, clip: float = 1.0, with_rot: bool = True):
    x = dev(x16)
    rows, d = x16.shape
    xr = torch.empty((rows, d), dtype=torch.float32, device="cuda") if with_rot else None
    q, s = qr.had_quant(x, dev(signs) if signs is not None else None, m, clip, x_rot_out=xr)
    return host(q), host(s), (host(xr) if with_rot else None)


_CACHE = {}


def act_inputs(name: str) -> dict:
    if name not in _CACHE:
        _CACHE.clear()
        _CACHE[name] = workloads.make_act_inputs(workloads.ACT_CONFIGS[name])
    return _CACHE[name]


# ---------------------------------------------------------------------------
# Fast transform against the dense matrix on small d
# ---------------------------------------------------------------------------
SMALL_D = [(32, 1), (64, 1), (128, 1), (256, 1), (512, 1), (1024, 1), (2048, 1), (4096, 1),
           (96, 12), (192, 12), (384, 12), (768, 12), (224, 28), (448, 28), (896, 28)]


@pytest.mark.parametrize("d,m", SMALL_D)
def test_rotation_equals_dense_hadamard(d, m):
    rng = np.random.default_rng(d + m)
    rows = 37
    x = rng.standard_normal((rows, d)).astype(np.float32)
    x[:, rng.integers(0, d)] *= 40.0
    x16 = x.astype(np.float16)
    signs = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    say(f"dense check d={d} m={m} rows={rows}")
    q, s, xr = gpu_had_quant(x16, signs, m)
    dense = oracle.dense_rotation(d, signs, m)
    ref = x16.astype(np.float64) @ dense.T
    check_rot(xr, ref, 1e-6)
    ref_q = oracle.had_quant(x16, signs, m)
    check_quant(oracle.unpack_int4(q), s, ref_q["x_rot"], ref_q["scales"])


# ---------------------------------------------------------------------------
# Rotate+quant on the configured workloads
# ---------------------------------------------------------------------------
ACT_SAMPLE = {"tiny": None, "llama7b_proj": 256, "down_12288": 64, "llama70b_down": 24}


@pytest.mark.parametrize("name", list(ACT_SAMPLE))
def test_had_quant_workload(name):
    cfg = workloads.ACT_CONFIGS[name]
    inp = act_inputs(name)
    x16 = inp["x"]
    say(f"had_quant {name}: x {x16.shape} m={cfg.m}")
    q, s, xr = gpu_had_quant(x16, inp["signs"], cfg.m)
    n = ACT_SAMPLE[name]
    rows = np.arange(x16.shape[0]) if n is None else np.unique(
        np.r_[0, x16.shape[0] - 1, np.random.default_rng(7).choice(x16.shape[0], n, replace=False)])
    ref = oracle.had_quant(x16[rows], inp["signs"], cfg.m)
    e = check_rot(xr[rows], ref["x_rot"])
    ns, f = check_quant(oracle.unpack_int4(q[rows]), s[rows], ref["x_rot"], ref["scales"])
    np.testing.assert_array_equal(oracle.pack_int4(oracle.unpack_int4(q[rows])), q[rows])
    say(f"  rows checked {len(rows)}: rot err {e:.2e}, scale ulps {ns}, code diff frac {f:.2e}")


def test_had_quant_weights_workload():
    # offline weight prep uses the same kernel on W's rows
    cfg = workloads.ACT_CONFIGS["llama7b_proj"]
    inp = act_inputs("llama7b_proj")
    w16 = inp["w"]
    say(f"had_quant weights: w {w16.shape}")
    q, s, xr = gpu_had_quant(w16, inp["signs"], cfg.m)
    rows = np.random.default_rng(11).choice(w16.shape[0], 128, replace=False)
    ref = oracle.prep_weights(w16[rows], inp["signs"], cfg.m)
    check_rot(xr[rows], ref["x_rot"])
    check_quant(oracle.unpack_int4(q[rows]), s[rows], ref["x_rot"], ref["scales"])


# ---------------------------------------------------------------------------
# GEMM fed the oracle's codes: bit-exact accumulators
# ---------------------------------------------------------------------------
GEMM_FED = [  # (workload, rows of X, rows of W)
    ("tiny", 16, 256),
    ("llama7b_proj", 200, 300),
    ("down_12288", 130, 260),
    ("llama70b_down", 72, 136),
]


@pytest.mark.parametrize("name,mr,nr", GEMM_FED)
def test_gemm_fed_oracle_codes(name, mr, nr):
    cfg = workloads.ACT_CONFIGS[name]
    inp = act_inputs(name)
    a = oracle.had_quant(inp["x"][:mr], inp["signs"], cfg.m)
    b = oracle.prep_weights(inp["w"][:nr], inp["signs"], cfg.m)
    acc_ref, y_ref = oracle.w4a4_reference(a["codes"], a["scales"], b["codes"], b["scales"])
    say(f"gemm fed oracle codes {name}: M={mr} N={nr} K={cfg.d}")
    acc = torch.empty((mr, nr), dtype=torch.int32, device="cuda")
    y = qr.w4a4_gemm(dev(a["packed"]), dev(a["scales"]), dev(b["packed"]), dev(b["scales"]),
                     cfg.d, acc_out=acc)
    np.testing.assert_array_equal(host(acc), acc_ref)
    check_y_elementwise(host(y), y_ref)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (33, 65, 96), (129, 257, 160), (256, 512, 384),
                                   (300, 700, 1056), (130, 260, 256), (64, 256, 512),
                                   (200, 300, 832), (128, 256, 1280), (257, 513, 1792)])
def test_gemm_ragged_shapes(M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    qa = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    qb = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    sa = (rng.uniform(0.01, 2.0, M)).astype(np.float16)
    sb = (rng.uniform(0.001, 0.1, N)).astype(np.float16)
    acc_ref, y_ref = oracle.w4a4_reference(qa, sa, qb, sb)
    say(f"gemm ragged M={M} N={N} K={K}")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = qr.w4a4_gemm(dev(oracle.pack_int4(qa)), dev(sa), dev(oracle.pack_int4(qb)), dev(sb), K,
                     acc_out=acc)
    np.testing.assert_array_equal(host(acc), acc_ref)
    check_y_elementwise(host(y), y_ref)


def test_gemm_extreme_codes():
    # all -8 x all -8 at K = 28672: acc = 64 K = 1835008 per output
    M, N, K = 64, 64, 28672
    qa = np.full((M, K), -8, np.int8)
    say("gemm extreme codes")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    ones = np.ones(M, np.float16)
    qr.w4a4_gemm(dev(oracle.pack_int4(qa)), dev(ones), dev(oracle.pack_int4(qa)), dev(ones), K,
                 acc_out=acc)
    assert np.all(host(acc) == 64 * K)


# The largest K the entry point takes (65536): 256 * |acc| reaches 2^30 for an
# all -8 row against an all -8 column, the widened accumulator's limit.  Ragged
# M and N on the eight-wave kernel, with extreme rows and columns among random
# ones; expected values from the oracle's integer GEMM.
def test_gemm_max_k_extreme_rows_ragged():
    M, N, K = 96, 300, 65536
    rng = np.random.default_rng(65536)
    qa = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    qb = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    qa[0] = -8
    qa[1] = 7
    qa[2, 0::2], qa[2, 1::2] = -8, 7
    qb[0] = -8
    qb[1] = 7
    qb[N - 1] = -8
    sa = rng.uniform(0.01, 1.0, M).astype(np.float16)
    sb = rng.uniform(0.001, 0.01, N).astype(np.float16)
    acc_ref, y_ref = oracle.w4a4_reference(qa, sa, qb, sb)
    assert acc_ref[0, 0] == 64 * K and acc_ref[1, 0] == -56 * K
    say(f"gemm max K M={M} N={N} K={K}")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = qr.w4a4_gemm(dev(oracle.pack_int4(qa)), dev(sa), dev(oracle.pack_int4(qb)), dev(sb), K,
                     acc_out=acc)
    np.testing.assert_array_equal(host(acc), acc_ref)
    check_y_elementwise(host(y), y_ref)


def test_gemm_large_tile_max_k_closed_form():
    # Large-tile kernel at K = 65536.  Rows of A and B are all -8, all 7, or
    # -8 at even and 7 at odd K, by index mod 3, so every accumulator has a
    # closed form: K/2 times 128, -112, 98, 8, -7 or 113 (the row types' dot
    # products over one even/odd pair).  Packed bytes follow the pages' layout
    # (even element in the low nibble): 0x88, 0x77 and 0x78.
    M, N, K = 4096, 4096, 65536
    pair = np.array([[128, -112, 8], [-112, 98, -7], [8, -7, 113]], np.int64)
    packed = np.array([0x88, 0x77, 0x78], np.uint8)
    ta, tb = np.arange(M) % 3, (np.arange(N) * 7 + 1) % 3
    a_q = np.repeat(packed[ta][:, None], K // 2, axis=1)
    b_q = np.repeat(packed[tb][:, None], K // 2, axis=1)
    acc_ref = pair[ta][:, tb] * (K // 2)
    assert acc_ref.max() == 64 * K and acc_ref.min() == -56 * K
    # scales 2^-8: y = acc / 2^16, every value exact in fp16
    sa = np.full(M, 2.0 ** -8, np.float16)
    sb = np.full(N, 2.0 ** -8, np.float16)
    say(f"gemm large tiles max K M={M} N={N} K={K}")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = qr.w4a4_gemm(dev(a_q), dev(sa), dev(b_q), dev(sb), K, acc_out=acc)
    np.testing.assert_array_equal(host(acc), acc_ref)
    np.testing.assert_array_equal(host(y).astype(np.float64), acc_ref / 65536.0)


# Shapes with at least 256 output tiles of 256 x 256 run the large-tile kernel
# (one wave per SIMD, 64-byte K tiles in a four-stage LDS ring): ragged M and
# N edges, a partial last K tile (K % 128 != 0) and an aligned case.
@pytest.mark.parametrize("M,N,K", [(4000, 4100, 1056), (4096, 4096, 2048), (3841, 4353, 672)])
def test_gemm_large_tile_shapes(M, N, K):
    rng = np.random.default_rng(M + 3 * N + 5 * K)
    qa = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    qb = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    sa = rng.uniform(0.01, 2.0, M).astype(np.float16)
    sb = rng.uniform(0.001, 0.1, N).astype(np.float16)
    assert ((M + 255) // 256) * ((N + 255) // 256) >= 256
    acc_ref, y_ref = oracle.w4a4_reference(qa, sa, qb, sb)
    say(f"gemm large tiles M={M} N={N} K={K}")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = qr.w4a4_gemm(dev(oracle.pack_int4(qa)), dev(sa), dev(oracle.pack_int4(qb)), dev(sb), K,
                     acc_out=acc)
    np.testing.assert_array_equal(host(acc), acc_ref)
    check_y_elementwise(host(y), y_ref)


# K shorter than the ring: no full K tile (the partial tile only), one, two
# or three full tiles, with the prologue's copies clamped to the last full tile.
@pytest.mark.parametrize("K", [32, 96, 128, 256, 384, 416])
def test_gemm_large_tile_short_k(K):
    M, N = 4096, 4112
    rng = np.random.default_rng(K)
    qa = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    qb = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    sa = rng.uniform(0.01, 2.0, M).astype(np.float16)
    sb = rng.uniform(0.001, 0.1, N).astype(np.float16)
    acc_ref, y_ref = oracle.w4a4_reference(qa, sa, qb, sb)
    say(f"gemm large tiles, short K: M={M} N={N} K={K}")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = qr.w4a4_gemm(dev(oracle.pack_int4(qa)), dev(sa), dev(oracle.pack_int4(qb)), dev(sb), K,
                     acc_out=acc)
    np.testing.assert_array_equal(host(acc), acc_ref)
    check_y_elementwise(host(y), y_ref)


def test_gemm_large_tile_strided_outputs():
    # the large-tile kernel's element-wise epilogue stores (ldc % 8 != 0,
    # accumulator row stride % 4 != 0) with ragged edges; guard bands past
    # each row stay untouched
    rng = np.random.default_rng(41)
    M, N, K = 4001, 4099, 800
    qa = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    qb = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    sa = rng.uniform(0.01, 2.0, M).astype(np.float16)
    sb = rng.uniform(0.001, 0.1, N).astype(np.float16)
    acc_ref, y_ref = oracle.w4a4_reference(qa, sa, qb, sb)
    say(f"gemm large tiles, strided outputs M={M} N={N} K={K}")
    ybuf = torch.full((M, N + 3), 7.0, dtype=torch.float16, device="cuda")
    abuf = torch.full((M, N + 5), -123, dtype=torch.int32, device="cuda")
    qr.w4a4_gemm(dev(oracle.pack_int4(qa)), dev(sa), dev(oracle.pack_int4(qb)), dev(sb), K,
                 out=ybuf[:, :N], acc_out=abuf[:, :N])
    yh, ah = host(ybuf), host(abuf)
    np.testing.assert_array_equal(ah[:, :N], acc_ref)
    assert np.all(ah[:, N:] == -123)
    assert np.all(yh[:, N:] == np.float16(7.0))
    check_y_elementwise(yh[:, :N], y_ref)


# Packed A and B rows inside wider buffers (lda, ldb > K/2, multiples of 16)
# whose padding bytes hold random codes: a read past the K/2 bytes of a row
# would add them to the sums.  Both the 64 x 64-tile and the large-tile kernel.
@pytest.mark.parametrize("M,N,K", [(300, 520, 800), (4000, 4100, 1056)])
def test_gemm_strided_inputs(M, N, K):
    rng = np.random.default_rng(M + N + K + 17)
    qa = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    qb = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    sa = rng.uniform(0.01, 2.0, M).astype(np.float16)
    sb = rng.uniform(0.001, 0.1, N).astype(np.float16)
    acc_ref, y_ref = oracle.w4a4_reference(qa, sa, qb, sb)
    lda, ldb = K // 2 + 16, K // 2 + 48
    abuf = rng.integers(0, 256, size=(M, lda), dtype=np.uint8)
    bbuf = rng.integers(0, 256, size=(N, ldb), dtype=np.uint8)
    abuf[:, : K // 2] = oracle.pack_int4(qa)
    bbuf[:, : K // 2] = oracle.pack_int4(qb)
    say(f"gemm strided inputs M={M} N={N} K={K} lda={lda} ldb={ldb}")
    a_dev, b_dev = dev(abuf)[:, : K // 2], dev(bbuf)[:, : K // 2]
    assert a_dev.stride(0) == lda and b_dev.stride(0) == ldb
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = qr.w4a4_gemm(a_dev, dev(sa), b_dev, dev(sb), K, acc_out=acc)
    np.testing.assert_array_equal(host(acc), acc_ref)
    check_y_elementwise(host(y), y_ref)


def test_gemm_large_tile_extreme_codes():
    # all -8 x all -8 at the 70B down-projection shape: acc = 64 K everywhere
    M, N, K = 4096, 4096, 28672
    qa = dev(oracle.pack_int4(np.full((1, K), -8, np.int8))).expand(M, K // 2).contiguous()
    say("gemm large-tile extreme codes M=N=4096 K=28672")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    ones = dev(np.ones(M, np.float16))
    qr.w4a4_gemm(qa, ones, qa, ones, K, acc_out=acc)
    assert bool((acc == 64 * K).all())


# ---------------------------------------------------------------------------
# Full-size pipelines, sampled: rotate X and W on the GPU, GEMM on the GPU
# ---------------------------------------------------------------------------
FULL = {"tiny": (16, 256), "llama7b_proj": (48, 64), "down_12288": (24, 48),
        "llama70b_down": (12, 24)}


@pytest.mark.parametrize("name", list(FULL))
def test_full_pipeline_sampled(name):
    cfg = workloads.ACT_CONFIGS[name]
    inp = act_inputs(name)
    x16, w16, signs = inp["x"], inp["w"], inp["signs"]
    say(f"full pipeline {name}: X {x16.shape} W {w16.shape}")
    xs = dev(signs)
    qx, sx = qr.had_quant(dev(x16), xs, cfg.m)
    qw, sw = qr.had_quant(dev(w16), xs, cfg.m)
    acc = torch.empty((x16.shape[0], w16.shape[0]), dtype=torch.int32, device="cuda")
    y = qr.w4a4_gemm(qx, sx, qw, sw, cfg.d, acc_out=acc)
    acc_h, y_h = host(acc), host(y)
    qx_h, sx_h, qw_h, sw_h = host(qx), host(sx), host(qw), host(sw)
    nr, nc = FULL[name]
    rng = np.random.default_rng(5)
    ri = np.unique(np.r_[0, x16.shape[0] - 1, rng.choice(x16.shape[0], nr, replace=False)])
    ci = np.unique(np.r_[0, w16.shape[0] - 1, rng.choice(w16.shape[0], nc, replace=False)])
    if name == "tiny":  # every row and column
        ri, ci = np.arange(x16.shape[0]), np.arange(w16.shape[0])
    # the GEMM is exact on whatever codes it was given
    cx = oracle.unpack_int4(qx_h[ri])
    cw = oracle.unpack_int4(qw_h[ci])
    np.testing.assert_array_equal(acc_h[np.ix_(ri, ci)], oracle.int_gemm_exact(cx, cw))
    # end to end against the oracle pipeline on the sampled rows and columns
    a = oracle.had_quant(x16[ri], signs, cfg.m)
    b = oracle.prep_weights(w16[ci], signs, cfg.m)
    check_quant(cx, sx_h[ri], a["x_rot"], a["scales"])
    check_quant(cw, sw_h[ci], b["x_rot"], b["scales"])
    _, y_ref = oracle.w4a4_reference(a["codes"], a["scales"], b["codes"], b["scales"])
    ys = y_h[np.ix_(ri, ci)]
    e = check_y_frobenius(ys, y_ref)
    same = (np.all(cx == a["codes"], axis=1)[:, None] & np.all(cw == b["codes"], axis=1)[None, :]
            & (sx_h[ri][:, None] == a["scales"][:, None]) & (sw_h[ci][None, :] == b["scales"][None, :]))
    check_y_elementwise(ys, y_ref, mask=same)
    say(f"  sampled {len(ri)}x{len(ci)}: frobenius {e:.2e}, exact-code cells {same.mean():.3f}")


# ---------------------------------------------------------------------------
# KV cache path
# ---------------------------------------------------------------------------
def test_kv_workload():
    # the full K/V launch, with the optional fp32 copy of every rotated group
    cfg = workloads.KV_CONFIG
    inp = workloads.make_kv_inputs(cfg)
    k16, v16, signs = inp["k"], inp["v"], inp["signs"]
    B, H, S, D = k16.shape
    say(f"kv {cfg.name}: K/V {k16.shape} with rotated outputs")
    kq = torch.empty((B, H, S, D // 2), dtype=torch.uint8, device="cuda")
    vq = torch.empty_like(kq)
    ks = torch.empty((B, H, S), dtype=torch.float16, device="cuda")
    vs = torch.empty_like(ks)
    kr = torch.empty((B, H, S, D), dtype=torch.float32, device="cuda")
    vr = torch.empty_like(kr)
    qr.kv_had_quant(dev(k16), dev(v16), dev(signs), kq, ks, vq, vs, pos0=0, k_rot_out=kr,
                    v_rot_out=vr)
    rng = np.random.default_rng(3)
    flat = np.unique(np.r_[0, B * H * S - 1, rng.choice(B * H * S, 4096, replace=False)])
    for t16, q_t, s_t, r_t, nm in ((k16, kq, ks, kr, "K"), (v16, vq, vs, vr, "V")):
        q_h, s_h = host(q_t), host(s_t)
        r_h = host(r_t).reshape(-1, D)[flat]
        rows = t16.reshape(-1, D)[flat]
        ref = oracle.had_quant(rows, signs, 1)
        e = check_rot(r_h, ref["x_rot"])
        _, f = check_quant(oracle.unpack_int4(q_h.reshape(-1, D // 2)[flat]), s_h.reshape(-1)[flat],
                           ref["x_rot"], ref["scales"])
        say(f"  {nm}: {len(flat)} groups sampled, rot err {e:.2e}, code diff frac {f:.2e}")
    del kr, vr


def test_kv_append_single_position():
    # decode-time append: S = 1 at pos0 = t writes cache position t only
    rng = np.random.default_rng(23)
    B, H, D, S_cache = 4, 8, 128, 96
    for t in (0, 41, S_cache - 1):
        k1 = rng.standard_normal((B, H, 1, D)).astype(np.float16)
        v1 = rng.standard_normal((B, H, 1, D)).astype(np.float16)
        signs = (1 - 2 * rng.integers(0, 2, D)).astype(np.int8)
        say(f"kv append S=1 at pos0={t}")
        kq = torch.full((B, H, S_cache, D // 2), 0x3C, dtype=torch.uint8, device="cuda")
        vq = torch.full_like(kq, 0xC3)
        ks = torch.full((B, H, S_cache), -1.0, dtype=torch.float16, device="cuda")
        vs = torch.full_like(ks, -2.0)
        qr.kv_had_quant(dev(k1), dev(v1), dev(signs), kq, ks, vq, vs, pos0=t)
        for src, q_t, s_t, fq, fs in ((k1, kq, ks, 0x3C, -1.0), (v1, vq, vs, 0xC3, -2.0)):
            q_h, s_h = host(q_t), host(s_t)
            ref = oracle.had_quant(src.reshape(-1, D), signs, 1)
            check_quant(oracle.unpack_int4(q_h[:, :, t].reshape(-1, D // 2)),
                        s_h[:, :, t].reshape(-1), ref["x_rot"], ref["scales"])
            keep = np.ones(S_cache, bool)
            keep[t] = False
            assert np.all(q_h[:, :, keep] == fq) and np.all(s_h[:, :, keep] == fs)


def test_kv_positions_strides_and_per_head_signs():
    rng = np.random.default_rng(21)
    B, H, S, D, S_cache, pos0 = 3, 4, 37, 128, 64, 19
    # K stored as [B, S, H, D] and viewed as [B, H, S, D] (non-contiguous)
    k_bshd = rng.standard_normal((B, S, H, D)).astype(np.float16)
    v_bshd = rng.standard_normal((B, S, H, D)).astype(np.float16)
    signs = (1 - 2 * rng.integers(0, 2, (H, D))).astype(np.int8)
    say("kv positions/strides/per-head signs")
    k_t = dev(k_bshd).permute(0, 2, 1, 3)
    v_t = dev(v_bshd).permute(0, 2, 1, 3)
    kq = torch.full((B, H, S_cache, D // 2), 0xAB, dtype=torch.uint8, device="cuda")
    vq = torch.full_like(kq, 0xCD)
    ks = torch.full((B, H, S_cache), -1.0, dtype=torch.float16, device="cuda")
    vs = torch.full_like(ks, -2.0)
    qr.kv_had_quant(k_t, v_t, dev(signs), kq, ks, vq, vs, pos0=pos0, signs_stride_h=D)
    kq_h, vq_h, ks_h, vs_h = host(kq), host(vq), host(ks), host(vs)
    for src, q_h, s_h, fill_q, fill_s in ((k_bshd, kq_h, ks_h, 0xAB, -1.0),
                                          (v_bshd, vq_h, vs_h, 0xCD, -2.0)):
        for h in range(H):
            rows = src[:, :, h, :].reshape(-1, D)
            ref = oracle.had_quant(rows, signs[h], 1)
            got_q = q_h[:, h, pos0:pos0 + S].reshape(-1, D // 2)
            got_s = s_h[:, h, pos0:pos0 + S].reshape(-1)
            check_quant(oracle.unpack_int4(got_q), got_s, ref["x_rot"], ref["scales"])
        # cache entries outside [pos0, pos0 + S) untouched
        assert np.all(q_h[:, :, :pos0] == fill_q) and np.all(q_h[:, :, pos0 + S:] == fill_q)
        assert np.all(s_h[:, :, :pos0] == fill_s) and np.all(s_h[:, :, pos0 + S:] == fill_s)


@pytest.mark.parametrize("mode", [0, 1])
def test_kv_block_aligned_strides_positions_and_per_head_signs(mode):
    # S a multiple of 128: each block's groups share (b, h), taken once per
    # block; strided [B, S, H, D] sources, a cache offset and per-head signs
    rng = np.random.default_rng(31 + mode)
    B, H, S, D, S_cache, pos0 = 2, 3, 256, 128, 300, 29
    k_bshd = rng.standard_normal((B, S, H, D)).astype(np.float16)
    v_bshd = (rng.standard_normal((B, S, H, D)) + 0.5).astype(np.float16)
    signs = (1 - 2 * rng.integers(0, 2, (H, D))).astype(np.int8)
    say(f"kv block-aligned S={S} mode={mode}")
    k_t = dev(k_bshd).permute(0, 2, 1, 3)
    v_t = dev(v_bshd).permute(0, 2, 1, 3)
    if mode == 1:
        out = gpu_kv_asym(k_bshd.transpose(0, 2, 1, 3), v_bshd.transpose(0, 2, 1, 3), signs,
                          0.95, S_cache=S_cache, pos0=pos0, signs_stride_h=D, k_t=k_t, v_t=v_t)
    else:
        kq = torch.full((B, H, S_cache, D // 2), 0x5A, dtype=torch.uint8, device="cuda")
        vq = torch.full_like(kq, 0x5A)
        ks = torch.full((B, H, S_cache), -3.0, dtype=torch.float16, device="cuda")
        vs = torch.full_like(ks, -3.0)
        qr.kv_had_quant(k_t, v_t, dev(signs), kq, ks, vq, vs, pos0=pos0, signs_stride_h=D)
        out = {"k": (host(kq), host(ks), None), "v": (host(vq), host(vs), None)}
    for src, nm in ((k_bshd, "k"), (v_bshd, "v")):
        q_h, s_h, z_h = out[nm]
        for h in range(H):
            rows = src[:, :, h, :].reshape(-1, D)
            got_q = q_h[:, h, pos0:pos0 + S].reshape(-1, D // 2)
            if mode == 1:
                x_rot = oracle.rotate_rows(rows, signs[h], 1)
                _, sc, zz = oracle.quantize_rows_asym(x_rot, 0.95)
                check_asym(oracle.unpack_uint4(got_q), s_h[:, h, pos0:pos0 + S],
                           z_h[:, h, pos0:pos0 + S], x_rot, {"scales": sc, "zeros": zz}, 0.95)
            else:
                ref = oracle.had_quant(rows, signs[h], 1)
                check_quant(oracle.unpack_int4(got_q), s_h[:, h, pos0:pos0 + S].reshape(-1),
                            ref["x_rot"], ref["scales"])
        # cache entries outside [pos0, pos0 + S) untouched
        assert np.all(q_h[:, :, :pos0] == 0x5A) and np.all(q_h[:, :, pos0 + S:] == 0x5A)
        assert np.all(s_h[:, :, :pos0] == -3.0) and np.all(s_h[:, :, pos0 + S:] == -3.0)


def test_kv_single_tensor_and_head_dims():
    rng = np.random.default_rng(4)
    for D in (32, 64, 128, 256):
        B, H, S = 2, 3, 11
        v16 = rng.standard_normal((B, H, S, D)).astype(np.float16)
        signs = (1 - 2 * rng.integers(0, 2, D)).astype(np.int8)
        say(f"kv V only D={D}")
        vq = torch.empty((B, H, S, D // 2), dtype=torch.uint8, device="cuda")
        vs = torch.empty((B, H, S), dtype=torch.float16, device="cuda")
        qr.kv_had_quant(None, dev(v16), dev(signs), None, None, vq, vs)
        ref = oracle.had_quant(v16.reshape(-1, D), signs, 1)
        check_quant(oracle.unpack_int4(host(vq).reshape(-1, D // 2)), host(vs).reshape(-1),
                    ref["x_rot"], ref["scales"])


# ---------------------------------------------------------------------------
# Edge cases of rotate+quant
# ---------------------------------------------------------------------------
def test_had_quant_strided_rows_clip_and_zero_rows():
    rng = np.random.default_rng(9)
    rows, d, ld = 45, 4096, 4096 + 64
    buf = rng.standard_normal((rows, ld)).astype(np.float16)
    buf[3] = 0  # an all-zero row
    signs = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    say("had_quant strided rows, clip 0.9, zero row")
    xt = dev(buf)[:, :d]
    qbuf = torch.full((rows, d // 2 + 32), 0x5A, dtype=torch.uint8, device="cuda")
    q_view = qbuf[:, : d // 2]
    s = torch.empty(rows, dtype=torch.float16, device="cuda")
    qr.had_quant(xt, dev(signs), 1, 0.9, q_out=q_view, scale_out=s)
    ref = oracle.had_quant(buf[:, :d], signs, 1, 0.9)
    qh = host(qbuf)
    assert np.all(qh[:, d // 2:] == 0x5A)
    check_quant(oracle.unpack_int4(qh[:, : d // 2]), host(s), ref["x_rot"], ref["scales"])
    assert np.all(qh[3, : d // 2] == 0)


# Power-of-two rows past the d = 4096 kernel run the generic kernel, with up
# to 15 butterfly stages.  The oracle's rotation is taken in its Kronecker
# form: the Sylvester H_d equals H_{d/128} (x) H_128 in natural order, so
# m = 128 with the Sylvester H_128 as the small factor is the same rotation,
# built from small matrices (pinned on the CPU).
@pytest.mark.parametrize("d", [8192, 16384, 32768])
def test_had_quant_large_power_of_two(d):
    rng = np.random.default_rng(d)
    rows = 37
    x16 = rng.standard_normal((rows, d)).astype(np.float16)
    ch = rng.choice(d, max(1, d // 1000), replace=False)
    x16[:, ch] *= 40
    signs = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    say(f"had_quant power of two d={d} rows={rows}")
    q, s, xr = gpu_had_quant(x16, signs, 1)
    ref = oracle.had_quant(x16, signs, 128, 1.0, hm=oracle.sylvester(128))
    check_rot(xr, ref["x_rot"])
    check_quant(oracle.unpack_int4(q), s, ref["x_rot"], ref["scales"])


@pytest.mark.parametrize("d", [256, 4096])
def test_exact_ties_round_to_even(d):
    # rows whose rotated values sit exactly on k + 1/2 steps of the scale.
    # x~ is built first (entries (k + 1/2) S with S = 1/8 exactly, plus the
    # row maximum 7 S), then x = s * (H x~) / sqrt(d), exactly representable
    # in fp16; for d = 4^k the kernels' transform of x is then exact too, so
    # every such element is an exact tie of x~ / S and must round to even.
    rng = np.random.default_rng(d)
    rows = 64
    h = oracle.sylvester(d).astype(np.float64)
    signs = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    xt = np.zeros((rows, d))
    for r in range(rows):
        pos = rng.choice(d, 15, replace=False)
        xt[r, pos[0]] = 7 * 0.125 * (1 - 2 * (r & 1))
        xt[r, pos[1:]] = (rng.integers(-7, 7, 14) + 0.5) * 0.125
    x = (xt @ h) / np.sqrt(d) * signs[None, :]
    x16 = x.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), x), "input not exact in fp16"
    say(f"exact ties d={d}: {rows} rows x 14 ties")
    q, s, xr = gpu_had_quant(x16, signs, 1)
    ref = oracle.had_quant(x16, signs, 1)
    np.testing.assert_allclose(ref["x_rot"], xt, rtol=0, atol=1e-15)
    assert np.all(ref["scales"] == np.float16(0.125))
    np.testing.assert_array_equal(xr, xt)          # the kernel's transform is exact
    np.testing.assert_array_equal(s, ref["scales"])
    codes = oracle.unpack_int4(q)
    tie = np.abs(np.abs(xt / 0.125) % 1.0 - 0.5) == 0.0
    away = int((codes[tie] != ref["codes"][tie]).sum())
    say(f"  {int(tie.sum())} ties, {away} rounded away from even")
    check_codes(codes, ref["codes"])
    assert away == 0


def test_had_quant_no_signs_single_row_and_determinism():
    rng = np.random.default_rng(12)
    for d, m in ((256, 1), (4096, 1), (12288, 12), (28672, 28)):
        x16 = rng.standard_normal((1, d)).astype(np.float16)
        say(f"had_quant single row no signs d={d}")
        q1, s1, _ = gpu_had_quant(x16, None, m, with_rot=False)
        q2, s2, _ = gpu_had_quant(x16, None, m, with_rot=False)
        np.testing.assert_array_equal(q1, q2)
        np.testing.assert_array_equal(s1, s2)
        ref = oracle.had_quant(x16, np.ones(d, np.int8), m)
        check_quant(oracle.unpack_int4(q1), s1, ref["x_rot"], ref["scales"])


@pytest.mark.parametrize("m", [12, 28])
@pytest.mark.parametrize("clip", [1.0, 0.9])
def test_had_quant_kron_rows_strided_grid_stride(m, clip):
    # d = 1024 m takes the Kronecker kernel; the rows exceed the blocks it
    # launches (two per compute unit for m = 12, one for m = 28), so blocks
    # walk several rows and prefetch the next one
    rng = np.random.default_rng(100 + m)
    d = 1024 * m
    rows, ld = (600 if m == 12 else 300), 1024 * m + 96
    buf = rng.standard_normal((rows, ld)).astype(np.float32)
    buf[:, rng.integers(0, d, 3)] *= 60.0
    buf = buf.astype(np.float16)
    buf[5] = 0
    signs = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    say(f"had_quant kron d={d} rows={rows} ld={ld} clip={clip}")
    xt = dev(buf)[:, :d]
    qbuf = torch.full((rows, d // 2 + 48), 0x5A, dtype=torch.uint8, device="cuda")
    s = torch.empty(rows, dtype=torch.float16, device="cuda")
    xr = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    qr.had_quant(xt, dev(signs), m, clip, q_out=qbuf[:, : d // 2], scale_out=s, x_rot_out=xr)
    ref = oracle.had_quant(buf[:, :d], signs, m, clip)
    qh = host(qbuf)
    assert np.all(qh[:, d // 2:] == 0x5A)
    check_rot(host(xr), ref["x_rot"])
    check_quant(oracle.unpack_int4(qh[:, : d // 2]), host(s), ref["x_rot"], ref["scales"])
    assert np.all(qh[5, : d // 2] == 0)


def test_gemm_strided_outputs():
    # output rows with ld % 8 != 0 and an accumulator row stride % 4 != 0 take
    # the element-wise epilogue stores; a guard band past each row must stay
    # untouched
    rng = np.random.default_rng(31)
    M, N, K = 150, 264, 768
    qa = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    qb = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    sa = rng.uniform(0.01, 2.0, M).astype(np.float16)
    sb = rng.uniform(0.001, 0.1, N).astype(np.float16)
    acc_ref, y_ref = oracle.w4a4_reference(qa, sa, qb, sb)
    say(f"gemm strided outputs M={M} N={N} K={K}")
    ybuf = torch.full((M, N + 3), 7.0, dtype=torch.float16, device="cuda")
    abuf = torch.full((M, N + 5), -123, dtype=torch.int32, device="cuda")
    qr.w4a4_gemm(dev(oracle.pack_int4(qa)), dev(sa), dev(oracle.pack_int4(qb)), dev(sb), K,
                 out=ybuf[:, :N], acc_out=abuf[:, :N])
    yh, ah = host(ybuf), host(abuf)
    np.testing.assert_array_equal(ah[:, :N], acc_ref)
    assert np.all(ah[:, N:] == -123)
    assert np.all(yh[:, N:] == np.float16(7.0))
    check_y_elementwise(yh[:, :N], y_ref)


# ---------------------------------------------------------------------------
# Asymmetric KV mode (zero point, uint4 codes)
# ---------------------------------------------------------------------------
def gpu_kv_asym(k16, v16, signs, clip, S_cache=None, pos0=0, signs_stride_h=0, k_t=None, v_t=None):
    B, H, S, D = k16.shape if k16 is not None else v16.shape
    S_cache = S if S_cache is None else S_cache
    out = {}
    bufs = []
    for nm in ("k", "v"):
        q = torch.full((B, H, S_cache, D // 2), 0x5A, dtype=torch.uint8, device="cuda")
        sc = torch.full((B, H, S_cache), -3.0, dtype=torch.float16, device="cuda")
        z = torch.full((B, H, S_cache), -5.0, dtype=torch.float16, device="cuda")
        bufs.append((q, sc, z))
    kt = k_t if k_t is not None else (dev(k16) if k16 is not None else None)
    vt = v_t if v_t is not None else (dev(v16) if v16 is not None else None)
    qr.kv_had_quant(kt, vt, dev(signs), bufs[0][0], bufs[0][1], bufs[1][0], bufs[1][1],
                    pos0=pos0, signs_stride_h=signs_stride_h, clip_ratio=clip, mode=1,
                    k_zero=bufs[0][2], v_zero=bufs[1][2])
    for nm, (q, sc, z) in zip(("k", "v"), bufs):
        out[nm] = (host(q), host(sc), host(z))
    return out


def test_kv_asym_workload():
    cfg = workloads.KV_CONFIG
    inp = workloads.make_kv_inputs(cfg, batch=2)
    k16, v16, signs = inp["k"], inp["v"], inp["signs"]
    B, H, S, D = k16.shape
    say(f"kv asym {cfg.name}: K/V {k16.shape} clip 0.95")
    out = gpu_kv_asym(k16, v16, signs, 0.95)
    for t16, nm in ((k16, "k"), (v16, "v")):
        q_h, s_h, z_h = out[nm]
        ref = oracle.kv_had_quant_asym(t16, signs, 0.95)
        g, f = check_asym(oracle.unpack_uint4(q_h.reshape(-1, D // 2)), s_h, z_h,
                          ref["x_rot"], ref, 0.95)
        say(f"  {nm}: {B * H * S} groups, (scale, zero) differ on {g:.2e}, codes {f:.2e}")


@pytest.mark.parametrize("D", [32, 64, 128, 256])
@pytest.mark.parametrize("clip", [1.0, 0.95])
def test_kv_asym_positions_heads_and_degenerate_groups(D, clip):
    rng = np.random.default_rng(40 + D)
    B, H, S, S_cache, pos0 = 2, 3, 21, 40, 11
    k_bshd = rng.standard_normal((B, S, H, D)).astype(np.float32)
    k_bshd[:, :, 1, :] += 4.0                       # a head with a large offset
    k_bshd = k_bshd.astype(np.float16)
    k_bshd[0, 2, 0, :] = 0                          # an all-zero group
    k_bshd[1, 3, 2, :] = np.float16(1.5)            # a constant group
    v_bshd = (np.abs(rng.standard_normal((B, S, H, D))) + 0.25).astype(np.float16)
    signs = (1 - 2 * rng.integers(0, 2, (H, D))).astype(np.int8)
    say(f"kv asym D={D} clip={clip} pos0={pos0}")
    k_t = dev(k_bshd).permute(0, 2, 1, 3)
    v_t = dev(v_bshd).permute(0, 2, 1, 3)
    out = gpu_kv_asym(k_bshd.transpose(0, 2, 1, 3), v_bshd.transpose(0, 2, 1, 3), signs, clip,
                      S_cache=S_cache, pos0=pos0, signs_stride_h=D, k_t=k_t, v_t=v_t)
    for src, nm in ((k_bshd, "k"), (v_bshd, "v")):
        q_h, s_h, z_h = out[nm]
        for h in range(H):
            rows = src[:, :, h, :].reshape(-1, D)
            x_rot = oracle.rotate_rows(rows, signs[h], 1)
            codes, sc, zz = oracle.quantize_rows_asym(x_rot, clip)
            ref = {"scales": sc, "zeros": zz}
            check_asym(oracle.unpack_uint4(q_h[:, h, pos0:pos0 + S].reshape(-1, D // 2)),
                       s_h[:, h, pos0:pos0 + S], z_h[:, h, pos0:pos0 + S], x_rot, ref, clip)
        assert np.all(q_h[:, :, :pos0] == 0x5A) and np.all(q_h[:, :, pos0 + S:] == 0x5A)
        assert np.all(s_h[:, :, :pos0] == -3.0) and np.all(z_h[:, :, pos0 + S:] == -5.0)
    # the zero and constant groups: scale from the 1e-5 floor, codes = the zero point
    q_h, s_h, z_h = out["k"]
    zg = oracle.unpack_uint4(q_h[0, 0, pos0 + 2])
    assert np.all(zg == int(z_h[0, 0, pos0 + 2])) and float(z_h[0, 0, pos0 + 2]) == 0.0
