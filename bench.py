#!/usr/bin/env python3
"""Benchmark of the rotated W4A4 hot path on one MI355X.

One step = one pass of the online path over one batch of synthetic input:
rotate+quant of the activations X (fused randomized Hadamard + per-token INT4,
``quarot_had_quant``) followed by the W4A4 GEMM with dequant
(``quarot_w4a4_gemm``) against weights prepared offline (untimed) by the same
rotate+quant kernel.  Default workload: the LLaMA-2-70B prefill
down-projection, X fp16 [4096 x 28672] (a SwiGLU-like product with 0.1%
outlier channels), random-sign H_1024 (x) H_28 (Paley), W int4
[8192 x 28672], Y fp16 [4096 x 8192].

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
Extra workloads for profiling: --workload NAME, --swiglu (the gated FFN
product fused into rotate+quant, against the unfused producer + rotate+quant),
--kv (the K/V cache write), --decode (one decode step: append the new token's
K/V, then attention of every query head over the int4 cache, with the
head-wise query rotation and the cross-head transform).
"""

from __future__ import annotations

import argparse
import json
import os
import re
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
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="llama70b_down", choices=sorted(workloads.ACT_CONFIGS))
    p.add_argument("--kv", action="store_true", help="benchmark the K/V cache write instead")
    p.add_argument("--kv-asym", action="store_true",
                   help="with --kv or --decode: the asymmetric cache (zero point, clip 0.95)")
    p.add_argument("--decode", action="store_true",
                   help="benchmark one decode step (append + attention over the int4 cache)")
    p.add_argument("--decode-workload", default="decode_70b_gqa",
                   choices=sorted(workloads.DECODE_CONFIGS))
    p.add_argument("--no-cross-head", action="store_true",
                   help="with --decode: leave out the cross-head transform")
    p.add_argument("--swiglu", action="store_true",
                   help="with a SwiGLU workload: rotate+quant fused with the gated product "
                        "SiLU(gate) * up, against the unfused producer + rotate+quant")
    p.add_argument("--cpu-rows", type=int, default=0,
                   help="token rows of the CPU oracle sample (0 = the workload's default)")
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


def time_kernel(torch, stream, launch, count: int, lead: int = 10) -> dict:
    """Per-launch duration (ms) of `count` back-to-back launches on `stream`.

    Two passes behind a spin kernel (so the host has enqueued everything
    before the first launch starts; `lead` untimed launches bring the clocks
    out of the spin's idle state):
      mean          two events around all launches of the first pass
      median, min   one event between consecutive launches of the second pass
    """
    def spin_and_lead():
        torch.cuda._sleep(SPIN_CYCLES)
        for i in range(lead):
            launch(i)

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    spin_and_lead()
    e0.record(stream)
    for i in range(count):
        launch(lead + i)
    e1.record(stream)
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) / count
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(count + 1)]
    spin_and_lead()
    evs[0].record(stream)
    for i in range(count):
        launch(lead + i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(count)]
    return {"mean": mean, "median": float(np.median(per)), "min": float(min(per))}


def us_stats(t: dict) -> dict:
    return {k: round(v * 1e3, 3) for k, v in t.items()}


# The source file each timed kernel is compiled from.
KERNEL_FILES = {"had_quant": "had_quant.hip", "swiglu_had_quant": "had_quant.hip",
                "w4a4_gemm": "gemm.hip",
                "kv_had_quant": "kv.hip", "kv_decode": "decode.hip",
                "cross_head": "cross_head.hip"}


def source_digest(kernel: str) -> str:
    """sha256 over a kernel's source file and the local headers it includes,
    transitively (the public header holds declarations only)."""
    import hashlib

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


def host_cpus() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# Token rows the CPU oracle times per workload: every token (each whole
# workload stays under about 10 s of host work on 16 cores).
CPU_ROWS = {"tiny": 16, "llama7b_proj": 2048, "down_12288": 2048, "llama70b_down": 4096}
# batch entries of the K/V cache write that the CPU oracle times (all of them)
KV_CPU_BATCH = 16


def cpu_baseline_act(cfg, inp, rows: int) -> dict:
    """The oracle, as it stands, on the first `rows` tokens of the step:
    rotate+quant of those rows, and their integer GEMM + dequant against all
    of W (whose offline preparation by the oracle is not timed)."""
    import oracle

    rows = min(rows, inp["x"].shape[0])
    x = inp["x"][:rows]
    t0 = time.perf_counter()
    a = oracle.had_quant(x, inp["signs"], cfg.m)
    t1 = time.perf_counter()
    b = oracle.prep_weights(inp["w"], inp["signs"], cfg.m)  # offline, not counted
    t2 = time.perf_counter()
    acc, y = oracle.w4a4_reference(a["codes"], a["scales"], b["codes"], b["scales"])
    t3 = time.perf_counter()
    d, N = cfg.d, inp["w"].shape[0]
    rq_bytes = 2 * rows * d + rows * d // 2 + 2 * rows
    return {
        "value": rq_bytes / (t1 - t0) / 1e9,
        "unit": "GB/s",
        "gemm_tops": 2.0 * rows * N * d / (t3 - t2) / 1e12,
        "seconds_rotate_quant": t1 - t0,
        "seconds_gemm_dequant": t3 - t2,
        "cores": blas_threads(),
        "host_cpus": host_cpus(),
        "kind": "oracle",
        "sample": f"{rows} of the {inp['x'].shape[0]} tokens of {cfg.name}: rotate+quant of "
                  f"X [{rows} x {d}] (float64 dense factored rotation, float64 rint) and the "
                  f"exact integer GEMM [{rows} x {N} x {d}] + dequant (float64 BLAS); the "
                  f"oracle's weight prep is not timed. cores = BLAS threads",
    }


def make_sets(n: int, make) -> list:
    return [make(i) for i in range(n)]


def bench_act(args, torch, qr) -> dict:
    cfg = workloads.ACT_CONFIGS[args.workload]
    log(f"workload {cfg.name}: generating inputs")
    inp = workloads.make_act_inputs(cfg)
    T, d, N = inp["x"].shape[0], cfg.d, inp["w"].shape[0]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    signs = dev(inp["signs"])
    had_m = qr.hadamard_factor(cfg.m) if cfg.m > 1 else None
    x0 = dev(inp["x"])
    w0 = dev(inp["w"])
    # offline weight prep (same kernel, untimed)
    qw0, sw0 = qr.had_quant(w0, signs, cfg.m, had_m=had_m)
    del w0
    per_set = T * d * 2 + T * d // 2 + 2 * T + N * d // 2 + 2 * N + T * N * 2
    nsets = args.sets or max(1, -(-CACHE_DEFEAT_BYTES // per_set))
    log(f"{nsets} buffer sets of {per_set / 2**20:.1f} MiB")
    sets = make_sets(nsets, lambda i: {
        "x": x0 if i == 0 else x0.clone(),
        "qx": torch.empty((T, d // 2), dtype=torch.uint8, device="cuda"),
        "sx": torch.empty((T,), dtype=torch.float16, device="cuda"),
        "qw": qw0 if i == 0 else qw0.clone(),
        "sw": sw0 if i == 0 else sw0.clone(),
        "y": torch.empty((T, N), dtype=torch.float16, device="cuda"),
    })
    stream = torch.cuda.current_stream()

    def rotate_quant(st):
        qr.had_quant(st["x"], signs, cfg.m, 1.0, q_out=st["qx"], scale_out=st["sx"],
                     had_m=had_m, stream=stream)

    def gemm(st):
        qr.w4a4_gemm(st["qx"], st["sx"], st["qw"], st["sw"], d, out=st["y"], stream=stream)

    def step(i):
        st = sets[i % nsets]
        rotate_quant(st)
        gemm(st)

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
    # (2) per-kernel durations from HIP events on the launch stream
    rq = time_kernel(torch, stream, lambda i: rotate_quant(sets[i % nsets]), args.steps)
    gm = time_kernel(torch, stream, lambda i: gemm(sets[i % nsets]), args.steps)
    rq_bytes = 2 * T * d + T * d // 2 + 2 * T
    gemm_ops = 2.0 * T * N * d
    rq_gbs = rq_bytes / (rq["mean"] * 1e-3) / 1e9
    tops = gemm_ops / (gm["mean"] * 1e-3) / 1e12
    log(f"rotate+quant {rq['mean'] * 1e3:.2f} us ({rq_gbs:.0f} GB/s); gemm "
        f"{gm['mean'] * 1e3:.2f} us ({tops:.0f} TOPS); wall/step {wall / args.steps * 1e3:.4f} ms")
    rot = f"H_{d // cfg.m}" + (f" (x) H_{cfg.m} (Paley)" if cfg.m > 1 else "")
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
            "workload": f"{cfg.name}: X fp16 [{T} x {d}]"
                        + (" (SiLU(A) * B)" if cfg.swiglu else "")
                        + f" with {cfg.outlier_count} outlier channels x U(10,100), rotation "
                        f"{rot} with random signs, W int4 [{N} x {d}], Y fp16 [{T} x {N}]",
            "tokens": T, "d": d, "n_out": N, "buffer_sets": nsets,
        },
        "kernels_us": {"had_quant": us_stats(rq), "w4a4_gemm": us_stats(gm)},
        "roofline": {
            "kernel": "w4a4_gemm",
            "bound": "mfma",
            "achieved": round(tops, 2),
            "peak": INT8_PEAK_TOPS,
            "unit": "TFLOP/s",
            "frac": round(tops / INT8_PEAK_TOPS, 4),
            "traffic": measured_traffic(cfg.name, "w4a4_gemm"),
            "note": "integer ops (TOPS) against the dense INT8 MFMA peak; 2*M*N*K per launch; "
                    "traffic = HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE",
        },
        "roofline_rotate_quant": {
            "kernel": "had_quant",
            "bound": "hbm",
            "achieved": round(rq_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(rq_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(cfg.name, "had_quant"),
            "algorithmic_bytes": rq_bytes,
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (baseline)")
        out["cpu_baseline"] = cpu_baseline_act(cfg, inp, args.cpu_rows or CPU_ROWS[cfg.name])
    return out


def bench_swiglu(args, torch, qr) -> dict:
    """The gated product fused into rotate+quant, against the same work
    unfused: torch's SiLU and multiply writing the fp16 product, then
    rotate+quant of it."""
    cfg = workloads.ACT_CONFIGS[args.workload]
    if not cfg.swiglu:
        raise SystemExit(f"--swiglu needs a SwiGLU workload, not {cfg.name}")
    log(f"swiglu workload {cfg.name}: generating inputs")
    inp = workloads.make_swiglu_inputs(cfg, with_w=False)
    T, d = inp["gate"].shape
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    signs = dev(inp["signs"])
    had_m = qr.hadamard_factor(cfg.m) if cfg.m > 1 else None
    g0, u0 = dev(inp["gate"]), dev(inp["up"])
    fused_bytes = 4 * T * d + T * d // 2 + 2 * T
    per_set = fused_bytes + 2 * T * d  # + the unfused product buffer
    nsets = args.sets or max(2, -(-CACHE_DEFEAT_BYTES // per_set))
    sets = make_sets(nsets, lambda i: {
        "g": g0 if i == 0 else g0.clone(), "u": u0 if i == 0 else u0.clone(),
        "x": torch.empty((T, d), dtype=torch.float16, device="cuda"),
        "q": torch.empty((T, d // 2), dtype=torch.uint8, device="cuda"),
        "s": torch.empty((T,), dtype=torch.float16, device="cuda")})
    stream = torch.cuda.current_stream()
    F = torch.nn.functional

    def fused(i):
        st = sets[i % nsets]
        qr.swiglu_had_quant(st["g"], st["u"], signs, cfg.m, 1.0, q_out=st["q"],
                            scale_out=st["s"], had_m=had_m, stream=stream)

    def producer(i):
        st = sets[i % nsets]
        torch.mul(F.silu(st["g"]), st["u"], out=st["x"])

    def unfused(i):
        producer(i)
        st = sets[i % nsets]
        qr.had_quant(st["x"], signs, cfg.m, 1.0, q_out=st["q"], scale_out=st["s"],
                     had_m=had_m, stream=stream)

    for i in range(args.warmup):
        fused(i)
        unfused(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fused(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tf = time_kernel(torch, stream, fused, args.steps)
    tu = time_kernel(torch, stream, unfused, args.steps)
    tp = time_kernel(torch, stream, producer, args.steps)
    gbs = fused_bytes / (tf["mean"] * 1e-3) / 1e9
    log(f"fused {tf['mean'] * 1e3:.2f} us ({gbs:.0f} GB/s); unfused {tu['mean'] * 1e3:.2f} us "
        f"(producer {tp['mean'] * 1e3:.2f} us)")
    out = {
        "metric": "gated product + rotate+quant GB/s (% HBM peak)",
        "value": round(gbs, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32 product and rotation (fp16 hi/lo MFMA operands) / int4 codes",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} gated product: gate, up fp16 [{T} x {d}], "
                               f"{cfg.outlier_count} outlier channels x U(10,100) in up, "
                               f"SiLU(gate) * up rotated by H_{d // cfg.m} (x) H_{cfg.m} with "
                               f"random signs, per-token int4",
                   "buffer_sets": nsets},
        "kernels_us": {"swiglu_had_quant": us_stats(tf),
                       "unfused_producer_plus_had_quant": us_stats(tu),
                       "unfused_producer_only": us_stats(tp)},
        "speedup_vs_unfused": round(tu["mean"] / tf["mean"], 3),
        "roofline": {"kernel": "swiglu_had_quant", "bound": "hbm", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(cfg.name + "_swiglu", "swiglu_had_quant"),
                     "algorithmic_bytes": fused_bytes},
    }
    if not args.no_cpu_baseline:
        import oracle

        rows = min(args.cpu_rows or CPU_ROWS[cfg.name], T)
        log("timing the CPU oracle on a sample")
        t0 = time.perf_counter()
        oracle.swiglu_had_quant(inp["gate"][:rows], inp["up"][:rows], inp["signs"], cfg.m)
        sec = time.perf_counter() - t0
        nb = rows * (4 * d + d // 2 + 2)
        out["cpu_baseline"] = {"value": nb / sec / 1e9, "unit": "GB/s", "seconds": sec,
                               "cores": blas_threads(), "host_cpus": host_cpus(),
                               "kind": "oracle",
                               "sample": f"{rows} of the {T} tokens (float64 SiLU product, "
                                         f"dense factored rotation, rint)"}
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
    tk = time_kernel(torch, stream, step, args.steps)
    ms = tk["mean"]
    nbytes = per_set
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"kv {ms * 1e3:.2f} us ({gbs:.0f} GB/s)")
    out = {
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
        "kernels_us": {"kv_had_quant": us_stats(tk)},
        "roofline": {"kernel": "kv_had_quant", "bound": "hbm", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(cfg.name + ("_asym" if asym else ""),
                                                 "kv_had_quant"),
                     "algorithmic_bytes": nbytes},
    }
    if not args.no_cpu_baseline:
        import oracle

        nb = min(KV_CPU_BATCH, B)
        log("timing the CPU oracle on a sample")
        t0 = time.perf_counter()
        for t in (inp["k"][:nb], inp["v"][:nb]):
            if asym:
                oracle.kv_had_quant_asym(t, inp["signs"], 0.95)
            else:
                oracle.kv_had_quant(t, inp["signs"])
        sec = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": per_set * nb / B / sec / 1e9, "unit": "GB/s",
                               "seconds": sec, "cores": blas_threads(),
                               "host_cpus": host_cpus(), "kind": "oracle",
                               "sample": f"K and V of {nb} of the {B} batch entries "
                                         f"(float64 H_{D} rotation, rint)"}
    return out


def cpu_baseline_cross_head(cfg, z16, rows=None) -> dict:
    """The oracle, as it stands, on the first ``rows`` tokens (default: all)."""
    import oracle

    rows = cfg.tokens if rows is None else rows
    t0 = time.perf_counter()
    oracle.cross_head_quant(z16[:rows], cfg.heads)
    dt = time.perf_counter() - t0
    nbytes = rows * (2 * cfg.d + cfg.d // 2 + 2)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "seconds": dt, "cores": blas_threads(),
            "host_cpus": host_cpus(), "kind": "oracle",
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
    tk = time_kernel(torch, stream, step, args.steps)
    ms = tk["mean"]
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
        "kernels_us": {"cross_head": us_stats(tk)},
        "roofline": {"kernel": "cross_head_quant", "bound": "hbm", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(cfg.name, "cross_head"),
                     "algorithmic_bytes": per_set},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline_cross_head(cfg, z16)
    return out


def cpu_baseline_decode(dcfg, inp, q16, mode: int, cross: bool, rows=None) -> dict:
    """The oracle, as it stands, on `rows` batch rows of the decode step
    (default: all of them; its cache built by the oracle's KV quantiser,
    untimed)."""
    import oracle
    from oracle.attention import decode_attention

    cfg = dcfg.kv
    rows = cfg.batch if rows is None else rows
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
            "host_cpus": host_cpus(), "kind": "oracle",
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
    t_step = time_kernel(torch, stream, step, args.steps)
    t_att = time_kernel(torch, stream, attend, args.steps)
    t_app = time_kernel(torch, stream, append, args.steps)
    ms_step, ms_att, ms_app = t_step["mean"], t_att["mean"], t_app["mean"]
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
        "kernels_us": {"kv_decode_attention": us_stats(t_att),
                       "kv_had_quant_append": us_stats(t_app), "decode_step": us_stats(t_step)},
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
# instantiations of the rotate+quant kernels that form the gated product first
GATED_KERNEL = re.compile(r"had_quant_kron<\d+, (?:true|false), true\b|"
                          r"had_quant_kront<\d+, (?:true|false), \d+, true\b|had_quant_lds<true>")


def kernel_key(kname: str):
    """Traffic key of a demangled kernel name, or None for kernels not tracked."""
    if "kv_had_quant" in kname:
        return "kv_had_quant"
    if "had_quant" in kname and GATED_KERNEL.search(kname):
        return "swiglu_had_quant"
    return next((v for k, v in KERNEL_KEYS.items() if k in kname), None)


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
            key = kernel_key(kname)
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
        elif args.swiglu:
            out = bench_swiglu(args, torch, qr)
        else:
            out = bench_act(args, torch, qr)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
