"""GPU parity of the gated FFN product fused into rotate+quant
(``quarot_swiglu_had_quant``) against ``oracle.swiglu_had_quant``.

"QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
summary), section 3.4 "FFN Activation Rotation (Stage 1b)": the online
Hadamard acts on c = SiLU(A) * B before the down-projection.  Inputs come
from ``workloads.make_swiglu_inputs`` (the gate and up projections of the
SwiGLU workloads) or from seeded generators here; expected values only from
``oracle``.  Rules in ``parity.py``.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from parity import check_codes, check_quant, check_rot, check_y_frobenius

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotated_w4a4_amd as qr  # noqa: E402


def say(msg: str) -> None:
    print(f"[swiglu] {msg}", flush=True)


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


SAMPLE = {"down_12288": 64, "llama70b_down": 24}


@pytest.mark.parametrize("name", list(SAMPLE))
def test_swiglu_workload_full_launch(name):
    # the whole workload in the benchmark's launch configuration, sampled rows
    cfg = workloads.ACT_CONFIGS[name]
    inp = workloads.make_swiglu_inputs(cfg, with_w=False)
    gate, up, signs = inp["gate"], inp["up"], inp["signs"]
    T, d = gate.shape
    say(f"{name}: gate/up {gate.shape} m={cfg.m}")
    xr = torch.empty((T, d), dtype=torch.float32, device="cuda")
    q, s = qr.swiglu_had_quant(dev(gate), dev(up), dev(signs), cfg.m, x_rot_out=xr)
    qh, sh, xh = host(q), host(s), host(xr)
    del xr
    rows = np.unique(np.r_[0, T - 1, np.random.default_rng(8).choice(T, SAMPLE[name],
                                                                     replace=False)])
    ref = oracle.swiglu_had_quant(gate[rows], up[rows], signs, cfg.m)
    e = check_rot(xh[rows], ref["x_rot"])
    ns, f = check_quant(oracle.unpack_int4(qh[rows]), sh[rows], ref["x_rot"], ref["scales"])
    say(f"  rows {len(rows)}: rot err {e:.2e}, scale ulps {ns}, code diff frac {f:.2e}")


def test_swiglu_pipeline_sampled():
    # fused rotate+quant of the gated product -> W4A4 GEMM against weights
    # prepared by the plain kernel; sampled rows and columns end to end
    cfg = workloads.ACT_CONFIGS["down_12288"]
    inp = workloads.make_swiglu_inputs(cfg)
    gate, up, w16, signs = inp["gate"], inp["up"], inp["w"], inp["signs"]
    say(f"pipeline down_12288: gate/up {gate.shape}, W {w16.shape}")
    xs = dev(signs)
    qx, sx = qr.swiglu_had_quant(dev(gate), dev(up), xs, cfg.m)
    qw, sw = qr.had_quant(dev(w16), xs, cfg.m)
    acc = torch.empty((gate.shape[0], w16.shape[0]), dtype=torch.int32, device="cuda")
    y = qr.w4a4_gemm(qx, sx, qw, sw, cfg.d, acc_out=acc)
    acc_h, y_h, qx_h, sx_h, qw_h, sw_h = (host(t) for t in (acc, y, qx, sx, qw, sw))
    rng = np.random.default_rng(6)
    ri = np.unique(np.r_[0, rng.choice(gate.shape[0], 24, replace=False)])
    ci = np.unique(np.r_[0, rng.choice(w16.shape[0], 48, replace=False)])
    cx, cw = oracle.unpack_int4(qx_h[ri]), oracle.unpack_int4(qw_h[ci])
    np.testing.assert_array_equal(acc_h[np.ix_(ri, ci)], oracle.int_gemm_exact(cx, cw))
    a = oracle.swiglu_had_quant(gate[ri], up[ri], signs, cfg.m)
    b = oracle.prep_weights(w16[ci], signs, cfg.m)
    check_quant(cx, sx_h[ri], a["x_rot"], a["scales"])
    check_quant(cw, sw_h[ci], b["x_rot"], b["scales"])
    _, y_ref = oracle.w4a4_reference(a["codes"], a["scales"], b["codes"], b["scales"])
    err = check_y_frobenius(y_h[np.ix_(ri, ci)], y_ref)
    say(f"  sampled {len(ri)}x{len(ci)}: frobenius {err:.2e}")


# d = 1024 m with m = 12, 28 run the Kronecker kernel (rows past the grid so
# blocks walk and prefetch several rows); the other shapes the generic kernel.
CASES = [(12288, 12, 600), (28672, 28, 300), (256, 1, 37), (4096, 1, 37), (1536, 12, 37),
         (640, 20, 21), (32768, 32, 5)]


@pytest.mark.parametrize("d,m,rows", CASES)
@pytest.mark.parametrize("clip", [1.0, 0.9])
def test_swiglu_shapes_strided_clip(d, m, rows, clip):
    rng = np.random.default_rng(d + m + rows + int(10 * clip))
    # gate and up interleaved in one buffer (a fused gate_up projection output
    # with padding): row r = [gate_r | up_r | pad], both strides 2 d + 64
    ld = 2 * d + 64
    buf = rng.standard_normal((rows, ld)).astype(np.float32)
    buf[:, d + rng.integers(0, d, 3)] *= 50.0  # outlier channels of up
    buf[:, rng.integers(0, d, 2)] = -30.0      # gate channels where SiLU ~ 0
    buf = buf.astype(np.float16)
    buf[3, :d] = 0                             # SiLU(0) = 0: an all-zero product row
    gate, up = buf[:, :d], buf[:, d:2 * d]
    signs = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    hm = oracle.hadamard_m(m) if m > 1 else None
    say(f"swiglu d={d} m={m} rows={rows} clip={clip} (strided gate/up)")
    b = dev(buf)
    qbuf = torch.full((rows, d // 2 + 32), 0x5A, dtype=torch.uint8, device="cuda")
    s = torch.empty(rows, dtype=torch.float16, device="cuda")
    xr = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    qr.swiglu_had_quant(b[:, :d], b[:, d:2 * d], dev(signs), m, clip, q_out=qbuf[:, : d // 2],
                        scale_out=s, x_rot_out=xr, had_m=hm)
    ref = oracle.swiglu_had_quant(gate, up, signs, m, clip, hm)
    qh = host(qbuf)
    assert np.all(qh[:, d // 2:] == 0x5A)
    e = check_rot(host(xr), ref["x_rot"])
    ns, f = check_quant(oracle.unpack_int4(qh[:, : d // 2]), host(s), ref["x_rot"],
                        ref["scales"])
    assert not qh[3, : d // 2].any()
    say(f"  rot err {e:.2e}, scale ulps {ns}, code diff frac {f:.2e}")


def test_swiglu_matches_plain_kernel_on_an_exact_product():
    # gate large enough that SiLU(gate) = gate in fp32 (exp underflows to 0)
    # and products exactly representable in fp16: the fused kernel must then
    # agree bit for bit with rotate+quant of the stored product
    rng = np.random.default_rng(3)
    for d, m in ((12288, 12), (28672, 28), (4096, 1)):
        rows = 40
        gate = np.full((rows, d), 128.0, np.float16)
        up = (rng.integers(-64, 65, (rows, d)) / 1024.0).astype(np.float16)
        prod = (gate.astype(np.float32) * up.astype(np.float32)).astype(np.float16)
        assert np.array_equal(prod.astype(np.float64), 128.0 * up.astype(np.float64))
        signs = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
        say(f"swiglu exact product d={d} m={m}")
        q1, s1 = qr.swiglu_had_quant(dev(gate), dev(up), dev(signs), m)
        q2, s2 = qr.had_quant(dev(prod), dev(signs), m)
        np.testing.assert_array_equal(host(s1), host(s2))
        check_codes(oracle.unpack_int4(host(q1)), oracle.unpack_int4(host(q2)))
