"""GPU parity of the decode attention over the INT4 cache, through the C ABI.

The caches are written by the oracle's KV quantiser from the seeded KV
recipe (``workloads.make_kv_inputs``); the queries from
``workloads.make_decode_query``.  Expected values come only from
``oracle.attention``; the comparison rule is ``parity.check_attention``.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import workloads
from oracle.attention import attend, cross_head, decode_attention, dequant_cache, rotate_heads
from parity import check_attention

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotated_w4a4_amd as qr  # noqa: E402


def say(msg: str) -> None:
    print(f"[decode] {msg}", flush=True)


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def oracle_cache(k16, v16, signs, mode):
    """The oracle's cache of K, V [B, H, S, 128]; signs [D] or [H, D]."""
    out = {}
    for name, t in (("k", k16), ("v", v16)):
        parts = []
        for h in range(t.shape[1]):
            s = signs if signs.ndim == 1 else signs[h]
            sl = t[:, h:h + 1]
            parts.append(oracle.kv_had_quant(sl, s) if mode == 0
                         else oracle.kv_had_quant_asym(sl, s, 0.95))
        out[f"{name}_q"] = np.concatenate([p["packed"] for p in parts], axis=1)
        out[f"{name}_scale"] = np.concatenate([p["scales"] for p in parts], axis=1)
        if mode == 1:
            z = np.concatenate([p["zeros"] for p in parts], axis=1)
            out[f"{name}_zero"] = z.astype(np.float16)
    return out


def expected(q16, signs, cache, lengths, mode, cross, sm_scale=None):
    """Oracle output and the magnitude sum_p p_p |v^_p| that scales its tolerance."""
    sm = 1.0 / math.sqrt(q16.shape[-1]) if sm_scale is None else sm_scale
    ref = decode_attention(q16, signs, cache, lengths, sm_scale=sm, mode=mode, cross=cross)
    k_hat = dequant_cache(cache["k_q"], cache["k_scale"], cache.get("k_zero"), mode)
    v_hat = dequant_cache(cache["v_q"], cache["v_scale"], cache.get("v_zero"), mode)
    q_rot = rotate_heads(q16, signs, k_hat.shape[1])
    mag = attend(q_rot, k_hat, np.abs(v_hat), lengths, sm)
    if cross:
        mag = np.repeat(mag.sum(axis=1, keepdims=True), mag.shape[1], axis=1) / math.sqrt(mag.shape[1])
    return ref, mag


def gpu_decode(q16, signs, cache, max_len, lengths, mode, cross, signs_stride_h=0, sm_scale=None):
    B, Hq, D = q16.shape
    out32 = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    out = qr.kv_decode_attention(
        dev(q16), dev(signs), dev(cache["k_q"]), dev(cache["k_scale"]), dev(cache["v_q"]),
        dev(cache["v_scale"]), max_len,
        lengths=dev(np.asarray(lengths, np.int32)) if lengths is not None else None,
        mode=mode, k_zero=dev(cache["k_zero"]) if mode == 1 else None,
        v_zero=dev(cache["v_zero"]) if mode == 1 else None, cross_head=cross,
        signs_stride_h=signs_stride_h, sm_scale=sm_scale, out_f32=out32)
    return host(out32), host(out)


# (B, Hkv, Hq, S_cache, max_len, lengths, mode, cross, per-head signs)
CASES = [
    (2, 2, 8, 300, 300, None, 0, False, False),          # ragged tail, group of 4
    (3, 1, 8, 1000, 777, [777, 1, 0], 0, True, False),   # lengths 1 and 0, cross-head
    (2, 4, 4, 640, 640, [640, 129], 1, False, True),     # zero-point cache, one head per group
    (1, 2, 16, 2048, 2048, None, 1, True, False),        # group of 8, cross-head over 16
    (4, 8, 8, 256, 200, [200, 50, 3, 17], 0, False, True),
    (2, 2, 6, 96, 96, [96, 95], 0, False, False),        # group of 3 (not a power of two)
    (1, 1, 1, 33, 33, None, 1, False, False),            # one head, 33 positions
    (2, 16, 128, 160, 160, [160, 77], 0, True, False),   # cross-head over 128 heads (LDS path)
    (2, 1, 2, 64, 64, None, 0, True, False),             # cross-head over 2 heads (lane path)
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_decode_against_oracle(case):
    B, Hkv, Hq, S_cache, max_len, lengths, mode, cross, per_head = case
    say(f"B={B} Hkv={Hkv} Hq={Hq} S_cache={S_cache} max_len={max_len} lengths={lengths} "
        f"mode={mode} cross={cross} per_head_signs={per_head}")
    cfg = workloads.KV_CONFIG
    inp = workloads.make_kv_inputs(cfg, seed=len(str(case)), batch=B, heads=Hkv, positions=S_cache)
    rng = np.random.default_rng(S_cache)
    signs = (np.stack([(1 - 2 * rng.integers(0, 2, 128)).astype(np.int8) for _ in range(Hkv)])
             if per_head else inp["signs"])
    cache = oracle_cache(inp["k"], inp["v"], signs, mode)
    q16 = workloads.make_decode_query(workloads.DecodeConfig("t", cfg, Hq), seed=S_cache, batch=B)
    lens = lengths if lengths is not None else [max_len] * B
    ref, mag = expected(q16, signs, cache, lens, mode, cross)
    got32, got16 = gpu_decode(q16, signs, cache, max_len, lengths, mode, cross,
                              signs_stride_h=128 if per_head else 0)
    err = check_attention(got32, got16, ref, mag)
    say(f"  max error {err:.2e} of the term magnitude")
    for b, n in enumerate(lens):
        if n <= 0 and not cross:
            assert not got32[b].any()


@pytest.mark.parametrize("mode", [0, 1])
def test_decode_flat_softmax(mode):
    """A tiny softmax scale spreads the weights over all 3000 positions, so
    the output is a near-average far smaller than its terms."""
    cfg = workloads.KV_CONFIG
    B, Hkv, Hq, S = 2, 2, 16, 3000
    say(f"flat softmax mode={mode} B={B} Hkv={Hkv} Hq={Hq} S={S}")
    inp = workloads.make_kv_inputs(cfg, seed=9, batch=B, heads=Hkv, positions=S)
    cache = oracle_cache(inp["k"], inp["v"], inp["signs"], mode)
    q16 = workloads.make_decode_query(workloads.DecodeConfig("t", cfg, Hq), seed=9, batch=B)
    ref, mag = expected(q16, inp["signs"], cache, [S, S], mode, True, sm_scale=1e-3)
    got32, got16 = gpu_decode(q16, inp["signs"], cache, S, None, mode, True, sm_scale=1e-3)
    err = check_attention(got32, got16, ref, mag)
    say(f"  max error {err:.2e} of the term magnitude (output / magnitude "
        f"{np.abs(ref).max() / mag.max():.3f})")


def test_decode_deterministic_and_workspace_reuse():
    """Bitwise-identical repeats on one workspace (filled with 0xFF first: its
    contents on entry do not matter), reused across shapes."""
    cfg = workloads.KV_CONFIG
    B, Hkv, Hq, S = 2, 2, 16, 700
    say(f"determinism B={B} Hkv={Hkv} Hq={Hq} S={S}")
    inp = workloads.make_kv_inputs(cfg, seed=5, batch=B, heads=Hkv, positions=S)
    cache = oracle_cache(inp["k"], inp["v"], inp["signs"], 0)
    q16 = workloads.make_decode_query(workloads.DecodeConfig("t", cfg, Hq), seed=5, batch=B)
    ws = torch.full((1 << 22,), 0xFF, dtype=torch.uint8, device="cuda")
    args = (dev(q16), dev(inp["signs"]), dev(cache["k_q"]), dev(cache["k_scale"]),
            dev(cache["v_q"]), dev(cache["v_scale"]), S)
    a = host(qr.kv_decode_attention(*args, workspace=ws, cross_head=True)).copy()
    b = host(qr.kv_decode_attention(*args, workspace=ws, cross_head=True))
    np.testing.assert_array_equal(a.view(np.uint16), b.view(np.uint16))
    # a different shape on the same workspace, then the first again
    say("  workspace reuse across shapes")
    B2, Hkv2, Hq2, S2 = 3, 4, 4, 300
    inp2 = workloads.make_kv_inputs(cfg, seed=6, batch=B2, heads=Hkv2, positions=S2)
    cache2 = oracle_cache(inp2["k"], inp2["v"], inp2["signs"], 0)
    q2 = workloads.make_decode_query(workloads.DecodeConfig("t", cfg, Hq2), seed=6, batch=B2)
    out2 = host(qr.kv_decode_attention(dev(q2), dev(inp2["signs"]), dev(cache2["k_q"]),
                                       dev(cache2["k_scale"]), dev(cache2["v_q"]),
                                       dev(cache2["v_scale"]), S2, workspace=ws))
    ref2, mag2 = expected(q2, inp2["signs"], cache2, [S2] * B2, 0, False)
    check_attention(out2.astype(np.float32), out2, ref2, mag2, tol=1e-3)
    c = host(qr.kv_decode_attention(*args, workspace=ws, cross_head=True))
    np.testing.assert_array_equal(a.view(np.uint16), c.view(np.uint16))


def test_decode_workload_sampled():
    """The 70B grouped-query shape in the launch configuration the benchmark
    times (16 x 8 KV heads x 4096 positions, 64 query heads): the oracle
    builds the cache of batch row 0 (all KV heads) and of three more sampled
    (batch, KV head) pairs, the other heads hold random codes.  Compared: the
    sampled pairs' query heads without the cross-head transform, and batch
    row 0 with it."""
    dcfg = workloads.DECODE_CONFIGS["decode_70b_gqa"]
    cfg = dcfg.kv
    B, Hkv, S, D, Hq = cfg.batch, cfg.heads, cfg.positions, cfg.head_dim, dcfg.q_heads
    say(f"decode workload {dcfg.name}: B={B} Hkv={Hkv} Hq={Hq} S={S}")
    inp = workloads.make_kv_inputs(cfg)
    rng = np.random.default_rng(7)
    cache = {"k_q": rng.integers(0, 256, (B, Hkv, S, D // 2), dtype=np.uint8),
             "v_q": rng.integers(0, 256, (B, Hkv, S, D // 2), dtype=np.uint8),
             "k_scale": rng.uniform(0.1, 1.0, (B, Hkv, S)).astype(np.float16),
             "v_scale": rng.uniform(0.1, 1.0, (B, Hkv, S)).astype(np.float16)}
    row0 = oracle_cache(inp["k"][:1], inp["v"][:1], inp["signs"], 0)
    for key in cache:
        cache[key][:1] = row0[key]
    pairs = [(0, 0), (0, 7), (5, 3), (11, 6), (15, 1)]
    for b, h in pairs[2:]:
        part = oracle_cache(inp["k"][b:b + 1, h:h + 1], inp["v"][b:b + 1, h:h + 1], inp["signs"], 0)
        for key in cache:
            cache[key][b, h] = part[key][0, 0]
    q16 = workloads.make_decode_query(dcfg)
    got32, got16 = gpu_decode(q16, inp["signs"], cache, S, None, 0, False)
    g = Hq // Hkv
    for b, h in pairs:
        sub = {k: v[b:b + 1, h:h + 1] for k, v in cache.items()}
        sl = slice(h * g, (h + 1) * g)
        ref, mag = expected(q16[b:b + 1, sl], inp["signs"], sub, [S], 0, False)
        err = check_attention(got32[b:b + 1, sl], got16[b:b + 1, sl], ref, mag)
        say(f"  pair (b={b}, kv={h}): max error {err:.2e} of the term magnitude")
    say("  batch row 0 with the cross-head transform over 64 heads")
    got32c, got16c = gpu_decode(q16, inp["signs"], cache, S, None, 0, True)
    ref, mag = expected(q16[:1], inp["signs"], {k: v[:1] for k, v in cache.items()}, [S], 0, True)
    err = check_attention(got32c[:1], got16c[:1], ref, mag)
    say(f"  row 0 cross-head: max error {err:.2e} of the term magnitude")
