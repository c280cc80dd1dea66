"""Seeded synthetic inputs for the rotated W4A4 hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation, no quantisation, no GEMM).  Both the CPU
oracle (under ``oracle/``) and the HIP path are fed from here, so the two
sides always see byte-identical inputs.

The recipes stand in for the activations the QuaRot pages measure on real
LLaMA-2 / Qwen3 checkpoints, which are not available here:

* "QuaRot Guide: Outlier-Free 4-Bit W4A4 LLM Quantization" (aifetchly blog),
  section "The Problem", item 2: about 0.1% of hidden channels carry
  magnitudes up to 100x the typical ones, always at the same channel indices.
* "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
  summary), section 3.4 "FFN Activation Rotation (Stage 1b)": the gated FFN
  product SiLU(A) * B feeds the down-projection and can re-create outliers.

Random draws (``numpy.random.default_rng(seed)``), in this fixed order:

* activation workloads: signs -> outlier channel indices -> outlier factors
  -> X -> W
* KV workload: signs -> K outlier lanes per head -> V outlier lanes per head
  -> K -> V

Every tensor handed to a kernel is fp16 (the weights too: a checkpoint stores
them in fp16; the offline rotation then works on that fp16 copy).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "ActConfig",
    "KVConfig",
    "ACT_CONFIGS",
    "KV_CONFIG",
    "make_act_inputs",
    "make_swiglu_inputs",
    "make_kv_inputs",
    "DecodeConfig",
    "DECODE_CONFIGS",
    "make_decode_query",
    "CrossHeadConfig",
    "CROSS_HEAD_CONFIGS",
    "make_attn_output",
    "random_signs",
    "config_by_name",
]


@dataclasses.dataclass(frozen=True)
class ActConfig:
    """A rotate+quant -> W4A4 GEMM workload: X [tokens x d], W [n_out x d]."""

    name: str
    tokens: int
    n: int  # log2 of the power-of-two factor of d
    m: int  # size of the small Hadamard factor (1 = pure power of two)
    n_out: int
    outlier_count: int  # number of fixed outlier channels
    outlier_lo: float  # outlier factors ~ U(lo, hi); lo == hi = constant factor
    outlier_hi: float
    swiglu: bool  # X = SiLU(A) * B instead of N(0, 1)
    w_std: float = 0.02

    @property
    def d(self) -> int:
        return (1 << self.n) * self.m


def _outlier_count(d: int) -> int:
    # 0.1% of the channels, at least one.
    return max(1, int(round(0.001 * d)))


ACT_CONFIGS = {
    # Tiny end-to-end case: 16 tokens x 256, one channel x 50, W 256 x 256.
    "tiny": ActConfig("tiny", 16, 8, 1, 256, 1, 50.0, 50.0, False),
    # LLaMA-7B-shaped projection input: 2048 x 4096, W 4096 x 4096.
    "llama7b_proj": ActConfig("llama7b_proj", 2048, 12, 1, 4096,
                              _outlier_count(4096), 10.0, 100.0, False),
    # Non-power-of-two down-projection: d = 12288 = 1024 * 12.
    "down_12288": ActConfig("down_12288", 2048, 10, 12, 4096,
                            _outlier_count(12288), 10.0, 100.0, True),
    # LLaMA-70B-shaped prefill down-projection: d = 28672 = 1024 * 28.
    "llama70b_down": ActConfig("llama70b_down", 4096, 10, 28, 8192,
                               _outlier_count(28672), 10.0, 100.0, True),
}


@dataclasses.dataclass(frozen=True)
class KVConfig:
    """K and V cache writes: fp16 [batch, heads, positions, head_dim]."""

    name: str
    batch: int
    heads: int
    positions: int
    head_dim: int
    lanes_per_head: int  # fixed outlier lanes per head
    factor: float


KV_CONFIG = KVConfig("kv_70b_gqa", 16, 8, 4096, 128, 2, 30.0)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """One decode step: the new query of every (batch row, query head) against
    a cache of ``kv.positions`` positions (the cache is the KV workload's)."""

    name: str
    kv: KVConfig
    q_heads: int


# LLaMA-2-70B-shaped grouped-query decode (8 KV heads, 64 query heads) on the
# KV workload's cache, and the LLaMA-2-7B attention of the pages' decode
# timing table (32 heads x 128, 2047 cached tokens + the new one, batch 16).
DECODE_CONFIGS = {
    "decode_70b_gqa": DecodeConfig("decode_70b_gqa", KV_CONFIG, 64),
    "decode_7b_mha": DecodeConfig("decode_7b_mha",
                                  KVConfig("kv_7b_mha", 16, 32, 2048, 128, 2, 30.0), 32),
}


def make_decode_query(cfg: DecodeConfig, seed: int = 0, batch: Optional[int] = None) -> np.ndarray:
    """Post-RoPE queries fp16 [batch, q_heads, head_dim] ~ N(0, 1), drawn from
    default_rng(seed + 1) so that the cache's own draws (default_rng(seed))
    stay those of the KV workload."""
    rng = np.random.default_rng(seed + 1)
    bsz = cfg.kv.batch if batch is None else batch
    q = rng.standard_normal((bsz, cfg.q_heads, cfg.kv.head_dim), dtype=np.float32)
    return q.astype(np.float16)


@dataclasses.dataclass(frozen=True)
class CrossHeadConfig:
    """Attention output Z [tokens x heads*head_dim] of a prefill, the input of
    the out-projection (cross-head transform, then per-token quantisation)."""

    name: str
    tokens: int
    heads: int
    head_dim: int
    loud_heads: int  # heads whose every lane is scaled by one U(10, 100) factor

    @property
    def d(self) -> int:
        return self.heads * self.head_dim


# LLaMA-2-7B (32 heads) and LLaMA-2-70B (64 heads) of 128 lanes, at the token
# counts of the activation workloads of the same models.
CROSS_HEAD_CONFIGS = {
    "attn_out_7b": CrossHeadConfig("attn_out_7b", 2048, 32, 128, 2),
    "attn_out_70b": CrossHeadConfig("attn_out_70b", 4096, 64, 128, 4),
}


def make_attn_output(cfg: CrossHeadConfig, seed: int = 0, tokens: Optional[int] = None) -> dict:
    """Z fp16 [tokens x heads*head_dim] ~ N(0, 1) with ``loud_heads`` heads
    (drawn without replacement) scaled by one U(10, 100) factor each: value
    vectors whose heads carry very different energies.  Draw order: loud
    heads -> their factors -> Z."""
    rng = np.random.default_rng(seed)
    t = cfg.tokens if tokens is None else tokens
    loud = np.sort(rng.choice(cfg.heads, size=cfg.loud_heads, replace=False))
    factors = rng.uniform(10.0, 100.0, size=cfg.loud_heads).astype(np.float32)
    z = rng.standard_normal((t, cfg.heads, cfg.head_dim), dtype=np.float32)
    z[:, loud, :] *= factors[None, :, None]
    return {"z": z.reshape(t, cfg.d).astype(np.float16), "loud_heads": loud,
            "loud_factors": factors}


def config_by_name(name: str):
    if name in ACT_CONFIGS:
        return ACT_CONFIGS[name]
    if name in CROSS_HEAD_CONFIGS:
        return CROSS_HEAD_CONFIGS[name]
    if name == KV_CONFIG.name:
        return KV_CONFIG
    if name in DECODE_CONFIGS:
        return DECODE_CONFIGS[name]
    raise KeyError(name)


def random_signs(rng: np.random.Generator, d: int) -> np.ndarray:
    """Rademacher vector in {-1, +1} as int8."""
    bits = rng.integers(0, 2, size=d, dtype=np.int8)
    return (1 - 2 * bits).astype(np.int8)


def _silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def make_act_inputs(cfg: ActConfig, seed: int = 0, tokens: Optional[int] = None,
                    n_out: Optional[int] = None, with_w: bool = True) -> dict:
    """Draw (signs, X fp16, W fp16) for an activation workload.

    ``tokens`` / ``n_out`` override the row counts (for small parity cases);
    the draw order and the recipe stay the same.
    """
    rng = np.random.default_rng(seed)
    d = cfg.d
    t = cfg.tokens if tokens is None else tokens
    no = cfg.n_out if n_out is None else n_out

    signs = random_signs(rng, d)
    idx = np.sort(rng.choice(d, size=cfg.outlier_count, replace=False))
    if cfg.outlier_lo == cfg.outlier_hi:
        factors = np.full(cfg.outlier_count, cfg.outlier_lo, dtype=np.float32)
    else:
        factors = rng.uniform(cfg.outlier_lo, cfg.outlier_hi,
                              size=cfg.outlier_count).astype(np.float32)
    if cfg.swiglu:
        a = rng.standard_normal((t, d), dtype=np.float32)
        b = rng.standard_normal((t, d), dtype=np.float32)
        x = _silu(a) * b
        del a, b
    else:
        x = rng.standard_normal((t, d), dtype=np.float32)
    x[:, idx] *= factors[None, :]
    x16 = x.astype(np.float16)
    del x
    out = {
        "signs": signs,
        "x": x16,
        "outlier_idx": idx,
        "outlier_factors": factors,
        "d": d,
        "n": cfg.n,
        "m": cfg.m,
    }
    if with_w:
        w = rng.standard_normal((no, d), dtype=np.float32) * np.float32(cfg.w_std)
        out["w"] = w.astype(np.float16)
    return out


def make_swiglu_inputs(cfg: ActConfig, seed: int = 0, tokens: Optional[int] = None,
                       n_out: Optional[int] = None, with_w: bool = True) -> dict:
    """Draw (signs, gate fp16, up fp16, W fp16) for the fused gated-product
    path of a SwiGLU workload: the two projections whose product SiLU(gate) *
    up is the workload's X.

    The draws are those of ``make_act_inputs`` (signs -> outlier indices ->
    outlier factors -> A -> B -> W): gate = fp16(A) and up = fp16(B) with the
    outlier channels of B multiplied by their factors, which scales the
    product's channels alike.  Signs and W equal make_act_inputs'.
    """
    if not cfg.swiglu:
        raise ValueError(f"{cfg.name} is not a gated-product workload")
    rng = np.random.default_rng(seed)
    d = cfg.d
    t = cfg.tokens if tokens is None else tokens
    no = cfg.n_out if n_out is None else n_out
    signs = random_signs(rng, d)
    idx = np.sort(rng.choice(d, size=cfg.outlier_count, replace=False))
    factors = rng.uniform(cfg.outlier_lo, cfg.outlier_hi, size=cfg.outlier_count).astype(np.float32)
    gate = rng.standard_normal((t, d), dtype=np.float32).astype(np.float16)
    up = rng.standard_normal((t, d), dtype=np.float32)
    up[:, idx] *= factors[None, :]
    out = {"signs": signs, "gate": gate, "up": up.astype(np.float16), "outlier_idx": idx,
           "outlier_factors": factors, "d": d, "n": cfg.n, "m": cfg.m}
    del up
    if with_w:
        w = rng.standard_normal((no, d), dtype=np.float32) * np.float32(cfg.w_std)
        out["w"] = w.astype(np.float16)
    return out


def make_kv_inputs(cfg: KVConfig = KV_CONFIG, seed: int = 0,
                   batch: Optional[int] = None, heads: Optional[int] = None,
                   positions: Optional[int] = None) -> dict:
    """Draw (signs, K fp16, V fp16) for the KV-cache write workload."""
    rng = np.random.default_rng(seed)
    bsz = cfg.batch if batch is None else batch
    nh = cfg.heads if heads is None else heads
    s = cfg.positions if positions is None else positions
    dh = cfg.head_dim

    signs = random_signs(rng, dh)
    k_lanes = np.stack([np.sort(rng.choice(dh, size=cfg.lanes_per_head, replace=False))
                        for _ in range(nh)])
    v_lanes = np.stack([np.sort(rng.choice(dh, size=cfg.lanes_per_head, replace=False))
                        for _ in range(nh)])
    k = rng.standard_normal((bsz, nh, s, dh), dtype=np.float32)
    v = rng.standard_normal((bsz, nh, s, dh), dtype=np.float32)
    for h in range(nh):
        k[:, h, :, k_lanes[h]] *= np.float32(cfg.factor)
        v[:, h, :, v_lanes[h]] *= np.float32(cfg.factor)
    return {
        "signs": signs,
        "k": k.astype(np.float16),
        "v": v.astype(np.float16),
        "k_lanes": k_lanes,
        "v_lanes": v_lanes,
    }


def log2_exact(v: int) -> int:
    n = int(math.log2(v))
    if (1 << n) != v:
        raise ValueError(f"{v} is not a power of two")
    return n
