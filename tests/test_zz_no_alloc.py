"""The allocation-free decode entry point (quarot_kv_decode_attention_noalloc)
against the existing one (quarot_kv_decode_attention with a workspace),
through the C ABI: two calls in a row, the second smaller, each compared with
the workspace call on the same inputs (bitwise: the same kernels run on the
same data) and the smaller one also with the oracle.  The library's scratch
array keeps the first call's partials when the second starts.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import workloads
from oracle.attention import attend, decode_attention, dequant_cache, rotate_heads
from parity import check_attention

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotated_w4a4_amd as qr  # noqa: E402


def say(msg: str) -> None:
    print(f"[noalloc] {msg}", flush=True)


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def make_case(B, Hkv, Hq, S, mode, seed):
    cfg = workloads.KV_CONFIG
    inp = workloads.make_kv_inputs(cfg, seed=seed, batch=B, heads=Hkv, positions=S)
    cache = {}
    for name in ("k", "v"):
        r = (oracle.kv_had_quant(inp[name], inp["signs"]) if mode == 0
             else oracle.kv_had_quant_asym(inp[name], inp["signs"], 0.95))
        cache[f"{name}_q"], cache[f"{name}_scale"] = r["packed"], r["scales"]
        if mode == 1:
            cache[f"{name}_zero"] = r["zeros"].astype(np.float16)
    q16 = workloads.make_decode_query(workloads.DecodeConfig("n", cfg, Hq), seed=seed, batch=B)
    return inp["signs"], cache, q16


def run(fn, signs, cache, q16, max_len, lengths, mode, cross, **kw):
    B, Hq, D = q16.shape
    out32 = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
    fn(dev(q16), dev(signs), dev(cache["k_q"]), dev(cache["k_scale"]), dev(cache["v_q"]),
       dev(cache["v_scale"]), max_len,
       lengths=dev(np.asarray(lengths, np.int32)) if lengths is not None else None, mode=mode,
       k_zero=dev(cache["k_zero"]) if mode == 1 else None,
       v_zero=dev(cache["v_zero"]) if mode == 1 else None, cross_head=cross, out=out,
       out_f32=out32, **kw)
    return host(out32), host(out)


# (B, Hkv, Hq, S_cache, max_len, lengths, mode, cross): the first fills most of
# the scratch's partials, the second is smaller
CALLS = [(8, 8, 64, 2048, 2048, None, 0, True),
         (2, 2, 8, 300, 300, [300, 41], 1, False)]


def test_noalloc_matches_workspace_entry_point_two_calls():
    for i, (B, Hkv, Hq, S, max_len, lengths, mode, cross) in enumerate(CALLS):
        need = qr.kv_decode_workspace_bytes(B, Hq, Hkv, 128, max_len)
        say(f"call {i}: B={B} Hkv={Hkv} Hq={Hq} S={S} mode={mode} cross={cross}, "
            f"partials {need} bytes")
        assert need <= 8 * 1024 * 1024
        signs, cache, q16 = make_case(B, Hkv, Hq, S, mode, seed=11 + i)
        g32, g16 = run(qr.kv_decode_attention_noalloc, signs, cache, q16, max_len, lengths,
                       mode, cross)
        w32, w16 = run(qr.kv_decode_attention, signs, cache, q16, max_len, lengths, mode, cross)
        assert not np.isnan(g32).any()
        np.testing.assert_array_equal(g32, w32)
        np.testing.assert_array_equal(g16, w16)
        if i == len(CALLS) - 1:
            lens = lengths if lengths is not None else [max_len] * B
            sm = 1.0 / math.sqrt(128)
            ref = decode_attention(q16, signs, cache, lens, sm_scale=sm, mode=mode, cross=cross)
            k_hat = dequant_cache(cache["k_q"], cache["k_scale"], cache.get("k_zero"), mode)
            v_hat = dequant_cache(cache["v_q"], cache["v_scale"], cache.get("v_zero"), mode)
            mag = attend(rotate_heads(q16, signs, Hkv), k_hat, np.abs(v_hat), lens, sm)
            err = check_attention(g32, g16, ref, mag)
            say(f"  against the oracle: {err:.2e} of the term magnitude")


def test_noalloc_rejects_sizes_past_its_scratch():
    B, Hkv, Hq, S = 256, 8, 64, 4096
    need = qr.kv_decode_workspace_bytes(B, Hq, Hkv, 128, S)
    assert need > 8 * 1024 * 1024
    say(f"sizes needing {need} bytes of partials are refused")
    u8, f16 = torch.uint8, torch.float16
    kq = torch.zeros((B, Hkv, S, 64), dtype=u8, device="cuda")
    ks = torch.zeros((B, Hkv, S), dtype=f16, device="cuda")
    q = torch.zeros((B, Hq, 128), dtype=f16, device="cuda")
    with pytest.raises(qr.QuarotError) as e:
        qr.kv_decode_attention_noalloc(q, None, kq, ks, kq, ks, S)
    assert e.value.status == -2
