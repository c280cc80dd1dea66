"""GPU parity of the RMSNorm-fused rotate+quant (quarot_rmsnorm_had_quant)
against the oracle, on every kernel path: the quad kernel (d <= 256), the
d = 4096 split kernel, the Kronecker kernels (d = 1024 m) and the generic
kernel.  Expected values come only from ``oracle.rmsnorm_had_quant``.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from parity import check_codes, check_rot, check_scales

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotated_w4a4_amd as qr  # noqa: E402


def say(msg: str) -> None:
    print(f"[rmsnorm] {msg}", flush=True)


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def run(x16, signs, m, clip, eps):
    rows, d = x16.shape
    xr = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    q, s = qr.rmsnorm_had_quant(dev(x16), eps, dev(signs), m, clip, x_rot_out=xr)
    ref = oracle.rmsnorm_had_quant(x16, signs, m, clip, eps)
    err = check_rot(host(xr), ref["x_rot"])
    check_scales(host(s), ref["scales"])
    f = check_codes(oracle.unpack_int4(host(q)), ref["codes"], frac=1e-2 if rows < 200 else 1e-3)
    return err, f


# (d, m): quad, split, Kronecker and generic paths
SHAPES = [(128, 1), (256, 1), (4096, 1), (12288, 12), (28672, 28), (512, 1), (768, 12), (1792, 28)]


@pytest.mark.parametrize("d,m", SHAPES)
@pytest.mark.parametrize("clip,eps", [(1.0, 1e-5), (0.9, 1e-6)])
def test_rmsnorm_had_quant_shapes(d, m, clip, eps):
    rng = np.random.default_rng(d + int(clip * 10))
    rows = 67
    # rows of very different magnitudes (the normalisation removes them),
    # one all-zero row, outlier channels
    x = rng.standard_normal((rows, d)) * np.exp(rng.uniform(-4, 4, (rows, 1)))
    x[:, rng.choice(d, max(1, d // 1000), replace=False)] *= 40.0
    x[5] = 0.0
    x16 = x.astype(np.float16)
    signs = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    say(f"d={d} m={m} clip={clip} eps={eps} rows={rows}")
    err, f = run(x16, signs, m, clip, eps)
    say(f"  rotated values max row-relative error {err:.2e}, code diff frac {f:.2e}")


@pytest.mark.parametrize("name", ["llama7b_proj", "down_12288"])
def test_rmsnorm_had_quant_workload_rows(name):
    """The workloads' rows (sampled to 512 tokens) through the fused path."""
    cfg = workloads.ACT_CONFIGS[name]
    inp = workloads.make_act_inputs(cfg, tokens=512, with_w=False)
    say(f"{name}: 512 x {cfg.d}")
    err, f = run(inp["x"], inp["signs"], cfg.m, 1.0, 1e-5)
    say(f"  rotated values max row-relative error {err:.2e}, code diff frac {f:.2e}")
