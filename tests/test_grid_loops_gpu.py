"""GPU parity of the launches whose grids are capped at 2^16 workgroups, at
sizes just past the cap, so that workgroups loop over further rows (groups):
rotate+quant at d = 32 (64 rows per workgroup pass), the KV path at D = 32
(64 groups per pass) and the cross-head transform (four rows per pass).
Sampled rows, among them the first ones of the second pass and the ragged
tail, are checked against the oracle; expected values come only from
``oracle``.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from parity import check_quant

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotated_w4a4_amd as qr  # noqa: E402

CAP = 1 << 16  # workgroups per grid pass


def say(msg: str) -> None:
    print(f"[grid_loops] {msg}", flush=True)


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def sample(n: int, per_pass: int, seed: int) -> np.ndarray:
    """Row indices: the first rows, rows around the end of the first grid
    pass, the tail, and a random spread."""
    rng = np.random.default_rng(seed)
    picks = [np.arange(64), np.arange(per_pass - 32, min(per_pass + 96, n)),
             np.arange(n - 64, n), rng.choice(n, 2048, replace=False)]
    return np.unique(np.concatenate(picks))


def test_had_quant_rows_past_grid_cap():
    d, per_pass = 32, CAP * 64
    rows = per_pass + 45
    rng = np.random.default_rng(61)
    x16 = (rng.standard_normal((rows, d), dtype=np.float32) * 2.0).astype(np.float16)
    signs = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    say(f"had_quant d={d} rows={rows} (grid pass {per_pass} rows)")
    q, s = qr.had_quant(dev(x16), dev(signs), 1)
    qh, sh = host(q), host(s)
    sel = sample(rows, per_pass, 1)
    ref = oracle.had_quant(x16[sel], signs, 1)
    check_quant(oracle.unpack_int4(qh[sel]), sh[sel], ref["x_rot"], ref["scales"])


def test_kv_groups_past_grid_cap():
    D, H, per_pass = 32, 2, CAP * 64
    S = per_pass // H + 77  # B * H * S groups = per_pass + 154
    rng = np.random.default_rng(62)
    v16 = (rng.standard_normal((1, H, S, D), dtype=np.float32) * 2.0).astype(np.float16)
    signs = (1 - 2 * rng.integers(0, 2, D)).astype(np.int8)
    say(f"kv D={D} H={H} S={S}: {H * S} groups (grid pass {per_pass} groups)")
    vq = torch.empty((1, H, S, D // 2), dtype=torch.uint8, device="cuda")
    vs = torch.empty((1, H, S), dtype=torch.float16, device="cuda")
    qr.kv_had_quant(None, dev(v16), dev(signs), None, None, vq, vs)
    groups = v16.reshape(-1, D)
    sel = sample(groups.shape[0], per_pass, 2)
    ref = oracle.had_quant(groups[sel], signs, 1)
    check_quant(oracle.unpack_int4(host(vq).reshape(-1, D // 2)[sel]), host(vs).reshape(-1)[sel],
                ref["x_rot"], ref["scales"])


def test_cross_head_rows_past_grid_cap():
    nh, per_pass = 2, CAP * 4
    rows = per_pass + 37
    rng = np.random.default_rng(63)
    z16 = (rng.standard_normal((rows, nh * 128), dtype=np.float32) * 2.0).astype(np.float16)
    say(f"cross-head n_heads={nh} rows={rows} (grid pass {per_pass} rows)")
    q, s = qr.cross_head_had_quant(dev(z16), nh)
    qh, sh = host(q), host(s)
    sel = sample(rows, per_pass, 3)
    ref = oracle.cross_head_quant(z16[sel], nh)
    check_quant(oracle.unpack_int4(qh[sel]), sh[sel], ref["x_rot"], ref["scales"])
