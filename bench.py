#!/usr/bin/env python3
"""Benchmark of the rotated W4A4 hot path on one MI355X.

One step = one pass of the online path over one batch of synthetic input:
rotate+quant of the activations X (fused randomized Hadamard + per-token INT4,
``quarot_had_quant``) followed by the W4A4 GEMM with dequant
(``quarot_w4a4_gemm``) against weights prepared offline (untimed) by the same
rotate+quant kernel.  Default workload: X fp16 [2048 x 4096] with 0.1%
outlier channels, random-sign H_4096, W int4 [4096 x 4096].

Inputs are resident in HBM before timing starts.  To keep the 256 MB
Infinity Cache from serving repeated reads, the step cycles over enough
independent buffer sets (inputs, weights and outputs) to exceed 1 GiB.

Prints ONE JSON line:
  value            rotate+quant algorithmic GB/s (fp16 read + int4 codes and
                   fp16 scales written), from HIP events around that kernel
  value_gemm_tops  GEMM algorithmic TOPS (2 M N K per launch)
  roofline         the dominant kernel (the GEMM) against INT8 MFMA peak
  roofline_rotate_quant  rotate+quant against HBM peak
  cpu_baseline     the CPU oracle timed on this host on the same workload
Extra workloads for profiling: --workload NAME, --kv (the K/V cache write),
--decode (one decode step: append the new token's K/V, then attention of every
query head over the int4 cache, with the head-wise query rotation and the
cross-head transform).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
CACHE_DEFEAT_BYTES = 1 << 30
SPIN_CYCLES = 200_000_000  # ~0.1 s of GPU spin before event-timed launches
CSRC = os.path.join(ROOT, "rotated_w4a4_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
COPY_BYTES = 256 << 20


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="llama7b_proj", choices=sorted(workloads.ACT_CONFIGS))
    p.add_argument("--kv", action="store_true", help="benchmark the K/V cache write instead")
    p.add_argument("--kv-asym", action="store_true",
                   help="with --kv or --decode: the asymmetric cache (zero point, clip 0.95)")
    p.add_argument("--decode", action="store_true",
                   help="benchmark one decode step (append + attention over the int4 cache)")
    p.add_argument("--decode-workload", default="decode_70b_gqa",
                   choices=sorted(workloads.DECODE_CONFIGS))
    p.add_argument("--no-cross-head", action="store_true",
                   help="with --decode: leave out the cross-head transform")
    p.add_argument("--rmsnorm", action="store_true",
                   help="with an activation workload: the RMSNorm-fused rotate+quant")
    p.add_argument("--cross-head", action="store_true",
                   help="benchmark the cross-head transform + quantisation of the attention output")
    p.add_argument("--cross-head-workload", default="attn_out_70b",
                   choices=sorted(workloads.CROSS_HEAD_CONFIGS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--sets", type=int, default=0, help="buffer sets (0 = enough for 1 GiB)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run a plain 256 MiB device copy (HBM counter calibration)")
    p.add_argument("--traffic-from", nargs="+", metavar="CSV",
                   help="write the HBM traffic summary from rocprofv3 --pmc CSVs: CAL_FETCH "
                        "CAL_WRITE, then WORKLOAD FETCH WRITE triples")
    return p.parse_args()


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def time_kernel(torch, stream, launch, count: int, lead: int = 10) -> float:
    """Average duration (ms) of `count` back-to-back launches on `stream`.

    A spin kernel holds the stream while the host enqueues everything, so no
    host launch latency lands between the events; `lead` untimed launches run
    right before the first event so the clocks have left the spin's idle
    state."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(SPIN_CYCLES)
    for i in range(lead):
        launch(i)
    e0.record(stream)
    for i in range(count):
        launch(lead + i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / count


# The source file each timed kernel is compiled from.
KERNEL_FILES = {"had_quant": "had_quant.hip", "w4a4_gemm": "gemm.hip",
                "kv_had_quant": "kv.hip", "kv_decode": "decode.hip",
                "cross_head": "cross_head.hip"}


def source_digest(kernel: str) -> str:
    """sha256 over a kernel's source file and the local headers it includes,
    transitively (the public header holds declarations only)."""
    import hashlib
    import re

    seen, todo = [], [KERNEL_FILES[kernel]]
    while todo:
        name = todo.pop()
        path = os.path.join(CSRC, name)
        if name in seen or not os.path.exists(path):
            continue
        seen.append(name)
        with open(path) as f:
            todo += re.findall(r'#include "([^"]+)"', f.read())
    h = hashlib.sha256()
    for name in sorted(seen):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel's sources changed since its counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(workload, {}).get(kernel)
    if not k or k.get("source_sha256") != source_digest(kernel):
        return None
    return int(k["fetch_bytes"] + k["write_bytes"])


def cpu_baseline_act(cfg, inp) -> dict:
    """The oracle, as it stands, on the full step of this workload."""
    import oracle

    t0 = time.perf_counter()
    a = oracle.had_quant(inp["x"], inp["signs"], cfg.m)
    t1 = time.perf_counter()
    b = oracle.prep_weights(inp["w"], inp["signs"], cfg.m)  # offline, not counted
    t2 = time.perf_counter()
    acc, y = oracle.w4a4_reference(a["codes"], a["scales"], b["codes"], b["scales"])
    t3 = time.perf_counter()
    T, d, N = inp["x"].shape[0], cfg.d, inp["w"].shape[0]
    rq_bytes = 2 * T * d + T * d // 2 + 2 * T
    return {
        "value": rq_bytes / (t1 - t0) / 1e9,
        "unit": "GB/s",
        "gemm_tops": 2.0 * T * N * d / (t3 - t2) / 1e12,
        "seconds_rotate_quant": t1 - t0,
        "seconds_gemm_dequant": t3 - t2,
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"full {cfg.name} step: rotate+quant of X [{T} x {d}] (float64 dense "
                  f"factored rotation) and the exact integer GEMM [{T} x {N} x {d}] + dequant "
                  f"(float64 BLAS); weight prep excluded",
    }


def bench_act(args, torch, qr) -> dict:
    cfg = workloads.ACT_CONFIGS[args.workload]
    log(f"workload {cfg.name}: generating inputs")
    inp = workloads.make_act_inputs(cfg)
    T, d, N = inp["x"].shape[0], cfg.d, inp["w"].shape[0]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    signs = dev(inp["signs"])
    x0 = dev(inp["x"])
    w0 = dev(inp["w"])
    # offline weight prep (same kernel, untimed)
    qw0, sw0 = qr.had_quant(w0, signs, cfg.m)
    del w0
    per_set = T * d * 2 + T * d // 2 + 2 * T + N * d // 2 + 2 * N + T * N * 2
    nsets = args.sets or max(1, -(-CACHE_DEFEAT_BYTES // per_set))
    log(f"{nsets} buffer sets of {per_set / 2**20:.1f} MiB")
    sets = []
    for _ in range(nsets):
        sets.append({
            "x": x0.clone(),
            "qx": torch.empty((T, d // 2), dtype=torch.uint8, device="cuda"),
            "sx": torch.empty((T,), dtype=torch.float16, device="cuda"),
            "qw": qw0.clone(),
            "sw": sw0.clone(),
            "y": torch.empty((T, N), dtype=torch.float16, device="cuda"),
        })
    stream = torch.cuda.current_stream()
    rms = args.rmsnorm

    def rotate_quant(s):
        if rms:
            qr.rmsnorm_had_quant(s["x"], 1e-5, signs, cfg.m, 1.0, q_out=s["qx"], scale_out=s["sx"],
                                 stream=stream)
        else:
            qr.had_quant(s["x"], signs, cfg.m, 1.0, q_out=s["qx"], scale_out=s["sx"], stream=stream)

    def step(i):
        s = sets[i % nsets]
        rotate_quant(s)
        qr.w4a4_gemm(s["qx"], s["sx"], s["qw"], s["sw"], d, out=s["y"], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup done; timing {args.steps} steps")
    # (1) the timed region: exactly K steps between two synchronisations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # (2) per-kernel durations from HIP events on the launch stream: K
    # back-to-back launches of one kernel (cycling over the buffer sets)
    # between two events, behind a spin kernel so the host has queued them
    # all before the first starts.
    def launch_rq(i):
        rotate_quant(sets[i % nsets])

    def launch_gemm(i):
        s = sets[i % nsets]
        qr.w4a4_gemm(s["qx"], s["sx"], s["qw"], s["sw"], d, out=s["y"], stream=stream)

    rq_ms = time_kernel(torch, stream, launch_rq, args.steps)
    gemm_ms = time_kernel(torch, stream, launch_gemm, args.steps)
    rq_bytes = 2 * T * d + T * d // 2 + 2 * T
    gemm_ops = 2.0 * T * N * d
    rq_gbs = rq_bytes / (rq_ms * 1e-3) / 1e9
    tops = gemm_ops / (gemm_ms * 1e-3) / 1e12
    log(f"rotate+quant {rq_ms * 1e3:.2f} us ({rq_gbs:.0f} GB/s); gemm {gemm_ms * 1e3:.2f} us "
        f"({tops:.0f} TOPS); wall/step {wall / args.steps * 1e3:.4f} ms")
    out = {
        "metric": "rotate+quant GB/s (% HBM peak); W4A4 GEMM TOPS (% INT8 MFMA peak)",
        "value": round(rq_gbs, 2),
        "unit": "GB/s",
        "value_gemm_tops": round(tops, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 rotate / int8 MFMA (int4 codes, int32 acc)",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: X fp16 [{T} x {d}] with {cfg.outlier_count} outlier "
                        f"channels, " + ("RMSNorm (eps 1e-5, gain absorbed) fused, " if rms else "")
                        + f"rotation H_{d // cfg.m}" + (f" (x) H_{cfg.m}" if cfg.m > 1 else "")
                        + f" with random signs, W int4 [{N} x {d}], Y fp16 [{T} x {N}]",
            "tokens": T, "d": d, "n_out": N, "buffer_sets": nsets,
        },
        "kernels_us": {"had_quant": round(rq_ms * 1e3, 3), "w4a4_gemm": round(gemm_ms * 1e3, 3)},
        "roofline": {
            "kernel": "w4a4_gemm",
            "bound": "mfma",
            "achieved": round(tops, 2),
            "peak": INT8_PEAK_TOPS,
            "unit": "TFLOP/s",
            "frac": round(tops / INT8_PEAK_TOPS, 4),
            "traffic": measured_traffic(cfg.name, "w4a4_gemm"),
            "note": "integer ops (TOPS) against the dense INT8 MFMA peak; 2*M*N*K per launch",
        },
        "roofline_rotate_quant": {
            "kernel": "rmsnorm_had_quant" if rms else "had_quant",
            "bound": "hbm",
            "achieved": round(rq_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(rq_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(cfg.name + ("_rmsnorm" if rms else ""), "had_quant"),
            "algorithmic_bytes": rq_bytes,
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (baseline)")
        out["cpu_baseline"] = cpu_baseline_act(cfg, inp)
    return out


def bench_kv(args, torch, qr) -> dict:
    cfg = workloads.KV_CONFIG
    log(f"kv workload {cfg.name}: generating inputs")
    inp = workloads.make_kv_inputs(cfg)
    B, H, S, D = inp["k"].shape
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    signs = dev(inp["signs"])
    k0, v0 = dev(inp["k"]), dev(inp["v"])
    asym = args.kv_asym
    per_set = 2 * (B * H * S * D * 2 + B * H * S * D // 2 + B * H * S * 2 * (2 if asym else 1))
    nsets = args.sets or max(2, -(-CACHE_DEFEAT_BYTES // per_set))
    sets = []
    for i in range(nsets):
        sets.append({
            "k": k0 if i == 0 else k0.clone(), "v": v0 if i == 0 else v0.clone(),
            "kq": torch.empty((B, H, S, D // 2), dtype=torch.uint8, device="cuda"),
            "vq": torch.empty((B, H, S, D // 2), dtype=torch.uint8, device="cuda"),
            "ks": torch.empty((B, H, S), dtype=torch.float16, device="cuda"),
            "vs": torch.empty((B, H, S), dtype=torch.float16, device="cuda"),
            "kz": torch.empty((B, H, S), dtype=torch.float16, device="cuda") if asym else None,
            "vz": torch.empty((B, H, S), dtype=torch.float16, device="cuda") if asym else None,
        })
    stream = torch.cuda.current_stream()

    def step(i):
        s = sets[i % nsets]
        if asym:
            qr.kv_had_quant(s["k"], s["v"], signs, s["kq"], s["ks"], s["vq"], s["vs"],
                            clip_ratio=0.95, mode=1, k_zero=s["kz"], v_zero=s["vz"], stream=stream)
        else:
            qr.kv_had_quant(s["k"], s["v"], signs, s["kq"], s["ks"], s["vq"], s["vs"],
                            stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = time_kernel(torch, stream, step, args.steps)
    nbytes = per_set
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"kv {ms * 1e3:.2f} us ({gbs:.0f} GB/s)")
    return {
        "metric": "KV rotate+quant GB/s (% HBM peak)" + (" [asymmetric, zero point]" if asym else ""),
        "value": round(gbs, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp32 rotate / int4 codes",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: K and V fp16 [{B} x {H} x {S} x {D}], "
                               f"H_{D} with random signs"
                               + (", asymmetric uint4 + fp16 scale and zero point, clip 0.95"
                                  if asym else ", symmetric int4 + fp16 scale"),
                   "buffer_sets": nsets},
        "roofline": {"kernel": "kv_had_quant", "bound": "hbm", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(cfg.name + ("_asym" if asym else ""),
                                                 "kv_had_quant"),
                     "algorithmic_bytes": nbytes},
    }


def cpu_baseline_cross_head(cfg, z16, rows=None) -> dict:
    """The oracle, as it stands, on the first ``rows`` tokens (default: all)."""
    import oracle

    rows = cfg.tokens if rows is None else rows
    t0 = time.perf_counter()
    oracle.cross_head_quant(z16[:rows], cfg.heads)
    dt = time.perf_counter() - t0
    nbytes = rows * (2 * cfg.d + cfg.d // 2 + 2)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "seconds": dt, "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{rows} of the {cfg.tokens} tokens of {cfg.name} (float64 einsum over the "
                      f"head index, then the quantiser)"}


def bench_cross_head(args, torch, qr) -> dict:
    cfg = workloads.CROSS_HEAD_CONFIGS[args.cross_head_workload]
    log(f"cross-head workload {cfg.name}: generating inputs")
    z16 = workloads.make_attn_output(cfg)["z"]
    T, d = z16.shape
    z0 = torch.from_numpy(z16).cuda()
    per_set = T * (2 * d + d // 2 + 2)
    nsets = args.sets or max(2, -(-CACHE_DEFEAT_BYTES // per_set))
    sets = []
    for i in range(nsets):
        sets.append({"z": z0 if i == 0 else z0.clone(),
                     "q": torch.empty((T, d // 2), dtype=torch.uint8, device="cuda"),
                     "s": torch.empty((T,), dtype=torch.float16, device="cuda")})
    stream = torch.cuda.current_stream()

    def step(i):
        st = sets[i % nsets]
        qr.cross_head_had_quant(st["z"], cfg.heads, 1.0, q_out=st["q"], scale_out=st["s"],
                                stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = time_kernel(torch, stream, step, args.steps)
    gbs = per_set / (ms * 1e-3) / 1e9
    log(f"cross-head {ms * 1e3:.2f} us ({gbs:.0f} GB/s)")
    out = {
        "metric": "cross-head transform + quant GB/s (% HBM peak)",
        "value": round(gbs, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp32 transform / int4 codes",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: attention output Z fp16 [{T} x {cfg.heads} x "
                               f"{cfg.head_dim}], {cfg.loud_heads} heads x U(10,100); "
                               f"H_{cfg.heads} over the head index, per-token int4",
                   "buffer_sets": nsets},
        "kernels_us": {"cross_head": round(ms * 1e3, 3)},
        "roofline": {"kernel": "cross_head_quant", "bound": "hbm", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(cfg.name, "cross_head"),
                     "algorithmic_bytes": per_set},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline_cross_head(cfg, z16)
    return out


def cpu_baseline_decode(dcfg, inp, q16, mode: int, cross: bool, rows: int = 4) -> dict:
    """The oracle, as it stands, on `rows` batch rows of the decode step (its
    cache built by the oracle's KV quantiser, untimed)."""
    import oracle
    from oracle.attention import decode_attention

    cfg = dcfg.kv
    S = cfg.positions
    quant = oracle.kv_had_quant if mode == 0 else (
        lambda t, s: oracle.kv_had_quant_asym(t, s, 0.95))
    kc, vc = quant(inp["k"][:rows], inp["signs"]), quant(inp["v"][:rows], inp["signs"])
    cache = {"k_q": kc["packed"], "k_scale": kc["scales"], "v_q": vc["packed"],
             "v_scale": vc["scales"]}
    if mode == 1:
        cache["k_zero"] = kc["zeros"].astype(np.float16)
        cache["v_zero"] = vc["zeros"].astype(np.float16)
    t0 = time.perf_counter()
    decode_attention(q16[:rows], inp["signs"], cache, [S] * rows, mode=mode, cross=cross)
    sec = time.perf_counter() - t0
    nbytes = decode_call_bytes(rows, cfg.heads, dcfg.q_heads, S, cfg.head_dim, mode)
    return {"value": nbytes / sec / 1e9, "unit": "GB/s", "seconds": sec, "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{rows} of {cfg.batch} batch rows of the decode attention (query rotation, "
                      f"dequantisation, float64 softmax attention{', cross-head' if cross else ''}) "
                      f"over {S} cached positions; the oracle's cache build is not timed"}


def decode_call_bytes(B, H, Hq, S, D, mode) -> int:
    """Algorithmic bytes of one decode attention call: every cached code, scale
    (and zero point) of K and V once, the queries read and the output written."""
    per_pos = D // 2 + 2 + (2 if mode == 1 else 0)
    return 2 * B * H * S * per_pos + 2 * B * Hq * D * 2


def bench_decode(args, torch, qr) -> dict:
    dcfg = workloads.DECODE_CONFIGS[args.decode_workload]
    cfg = dcfg.kv
    B, H, S, D, Hq = cfg.batch, cfg.heads, cfg.positions, cfg.head_dim, dcfg.q_heads
    mode = 1 if args.kv_asym else 0
    cross = not args.no_cross_head
    log(f"decode workload {dcfg.name}: generating inputs")
    inp = workloads.make_kv_inputs(cfg)
    q16 = workloads.make_decode_query(dcfg)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    signs = dev(inp["signs"])
    zero_kw = {"mode": 1, "clip_ratio": 0.95} if mode == 1 else {}

    def new_cache():
        c = {"kq": torch.empty((B, H, S, D // 2), dtype=torch.uint8, device="cuda"),
             "vq": torch.empty((B, H, S, D // 2), dtype=torch.uint8, device="cuda"),
             "ks": torch.empty((B, H, S), dtype=torch.float16, device="cuda"),
             "vs": torch.empty((B, H, S), dtype=torch.float16, device="cuda")}
        c["kz"] = torch.empty_like(c["ks"]) if mode == 1 else None
        c["vz"] = torch.empty_like(c["vs"]) if mode == 1 else None
        return c

    # the cache of all S positions, written by the library's KV quantiser; the
    # decode step re-appends position S - 1 (the new token) and attends to S
    k_all, v_all = dev(inp["k"]), dev(inp["v"])
    c0 = new_cache()
    qr.kv_had_quant(k_all, v_all, signs, c0["kq"], c0["ks"], c0["vq"], c0["vs"],
                    k_zero=c0["kz"], v_zero=c0["vz"], **zero_kw)
    k_new = k_all[:, :, S - 1:S].contiguous()
    v_new = v_all[:, :, S - 1:S].contiguous()
    del k_all, v_all
    att_bytes = decode_call_bytes(B, H, Hq, S, D, mode)
    app_bytes = 2 * B * H * (D * 2 + D // 2 + 2 + (2 if mode == 1 else 0))
    nsets = args.sets or max(2, -(-CACHE_DEFEAT_BYTES // att_bytes))
    sets = []
    for i in range(nsets):
        c = c0 if i == 0 else {k: (v.clone() if v is not None else None) for k, v in c0.items()}
        c["q"] = dev(q16)
        c["out"] = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
        sets.append(c)
    ws = torch.empty(qr.kv_decode_workspace_bytes(B, Hq, H, D, S), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def append(i):
        c = sets[i % nsets]
        qr.kv_had_quant(k_new, v_new, signs, c["kq"], c["ks"], c["vq"], c["vs"], pos0=S - 1,
                        k_zero=c["kz"], v_zero=c["vz"], stream=stream, **zero_kw)

    def attend(i):
        c = sets[i % nsets]
        qr.kv_decode_attention(c["q"], signs, c["kq"], c["ks"], c["vq"], c["vs"], S, mode=mode,
                               k_zero=c["kz"], v_zero=c["vz"], cross_head=cross, out=c["out"],
                               workspace=ws, stream=stream)

    def step(i):
        append(i)
        attend(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = time_kernel(torch, stream, step, args.steps)
    ms_att = time_kernel(torch, stream, attend, args.steps)
    ms_app = time_kernel(torch, stream, append, args.steps)
    step_gbs = (att_bytes + app_bytes) / (ms_step * 1e-3) / 1e9
    att_gbs = att_bytes / (ms_att * 1e-3) / 1e9
    log(f"decode step {ms_step * 1e3:.2f} us ({step_gbs:.0f} GB/s); attention call "
        f"{ms_att * 1e3:.2f} us ({att_gbs:.0f} GB/s); append {ms_app * 1e3:.2f} us")
    out = {
        "metric": "decode step GB/s (% HBM peak): append + attention over the int4 KV cache"
                  + (" [asymmetric, zero point]" if mode == 1 else ""),
        "value": round(step_gbs, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 cache, fp32-class attention (fp16 MFMA with hi/lo operand split)",
        "data": "synthetic",
        "config": {"workload": f"{dcfg.name}: q fp16 [{B} x {Hq} x {D}] against K and V caches "
                               f"[{B} x {H} x {S} x {D // 2}] uint8 + fp16 scales"
                               + (" + zero points" if mode == 1 else "")
                               + f", head-wise query rotation H_{D} with random signs"
                               + (f", cross-head H_{Hq}" if cross else ""),
                   "tokens_per_s": round(B / (ms_step * 1e-3), 1),
                   "buffer_sets": nsets},
        "kernels_us": {"kv_decode_attention": round(ms_att * 1e3, 3),
                       "kv_had_quant_append": round(ms_app * 1e3, 3)},
        "roofline": {"kernel": "kv_decode_attention (split + combine kernels)", "bound": "hbm",
                     "achieved": round(att_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(att_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(dcfg.name + ("_asym" if mode == 1 else ""),
                                                 "kv_decode"),
                     "algorithmic_bytes": att_bytes},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline_decode(dcfg, inp, q16, mode, cross)
    return out


def calibrate_copy(torch) -> dict:
    """A plain device copy of known size, for scaling the HBM byte counters."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "launches": 5}


def counter_means(path: str, counter: str, min_dispatches: int = 3) -> dict:
    """Median of one counter per kernel name in a rocprofv3 counter CSV.
    Kernels dispatched fewer than `min_dispatches` times (one-off launches
    such as the weight preparation) are left out."""
    import csv

    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: float(np.median(v)) for k, v in acc.items() if len(v) >= min_dispatches}


# kernel-name fragment -> traffic key; kernels sharing a key (the decode
# call's split and combine kernels) are summed
KERNEL_KEYS = {"w4a4_gemm": "w4a4_gemm", "had_quant": "had_quant", "kv_had_quant": "kv_had_quant",
               "decode_split": "kv_decode", "decode_combine": "kv_decode",
               "cross_head_quant": "cross_head"}


def summarize_counters(args) -> dict:
    """Build the HBM traffic summary from rocprofv3 --pmc runs.

    --traffic-from CAL_FETCH CAL_WRITE then, per workload, NAME FETCH WRITE
    (CSV paths).  FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by
    the ratio of known bytes to what the same counter reads for the plain
    copy kernel of the calibration run."""
    cal_f = counter_means(args.traffic_from[0], "FETCH_SIZE", 1)
    cal_w = counter_means(args.traffic_from[1], "WRITE_SIZE", 1)
    copy_f = max(v for k, v in cal_f.items() if "copy" in k.lower())
    copy_w = max(v for k, v in cal_w.items() if "copy" in k.lower())
    kf = COPY_BYTES / (copy_f * 1024.0)
    kw = COPY_BYTES / (copy_w * 1024.0)
    out = {"copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": copy_f, "write_kib": copy_w,
                                "fetch_scale": kf, "write_scale": kw},
           "kernels": {}}
    rest = args.traffic_from[2:]
    for i in range(0, len(rest), 3):
        name, fpath, wpath = rest[i:i + 3]
        f = counter_means(fpath, "FETCH_SIZE")
        w = counter_means(wpath, "WRITE_SIZE")
        ent = {}
        for kname, fv in f.items():
            key = next((v for k, v in KERNEL_KEYS.items() if k in kname and
                        not (k == "had_quant" and "kv_had_quant" in kname)), None)
            if key is None or kname not in w:
                continue
            e = ent.setdefault(key, {"kernel": "", "source_sha256": source_digest(key),
                                     "fetch_kib": 0.0, "write_kib": 0.0,
                                     "fetch_bytes": 0.0, "write_bytes": 0.0})
            short = kname.replace("(anonymous namespace)::", "").split("(")[0]
            e["kernel"] = (e["kernel"] + " + " if e["kernel"] else "") + short
            e["fetch_kib"] += fv
            e["write_kib"] += w[kname]
            e["fetch_bytes"] += fv * 1024.0 * kf
            e["write_bytes"] += w[kname] * 1024.0 * kw
        out["kernels"][name] = ent
    return out


def main() -> int:
    args = parse_args()
    if args.traffic_from:
        t = summarize_counters(args)
        # workloads not re-measured in this run keep their earlier entries
        if os.path.exists(TRAFFIC_FILE):
            with open(TRAFFIC_FILE) as f:
                old = json.load(f).get("kernels", {})
            for name, ent in old.items():
                t["kernels"].setdefault(name, ent)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path has no cross-GPU exchange; see the sharding notes)", file=sys.stderr)
        return 2
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    import rotated_w4a4_amd as qr

    qr.lib()
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        out = calibrate_copy(torch)
    else:
        if args.cross_head:
            out = bench_cross_head(args, torch, qr)
        elif args.decode:
            out = bench_decode(args, torch, qr)
        elif args.kv:
            out = bench_kv(args, torch, qr)
        else:
            out = bench_act(args, torch, qr)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
