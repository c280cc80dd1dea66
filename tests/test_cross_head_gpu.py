"""GPU parity of the cross-head transform + per-token quantisation
(quarot_cross_head_had_quant) against the oracle: every supported head count,
ragged row counts, clip < 1, strided input and output rows, an all-zero row,
the attention-output workloads' rows, and sampled rows of the full 70B-shaped
launch that the benchmark times.  Expected values come only from
``oracle.cross_head_quant``.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from parity import check_quant, check_rot

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotated_w4a4_amd as qr  # noqa: E402

DH = 128


def say(msg: str) -> None:
    print(f"[cross_head] {msg}", flush=True)


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check(z16, nh, clip, q, s, zr):
    ref = oracle.cross_head_quant(z16, nh, clip)
    err = check_rot(zr, ref["x_rot"])
    _, f = check_quant(oracle.unpack_int4(q), s, ref["x_rot"], ref["scales"])
    return err, f


@pytest.mark.parametrize("nh", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("clip", [1.0, 0.9])
def test_cross_head_head_counts(nh, clip):
    rng = np.random.default_rng(nh * 10 + int(clip * 10))
    rows = 67  # not a multiple of the four rows per workgroup
    z = rng.standard_normal((rows, nh, DH)) * np.exp(rng.uniform(-3, 3, (rows, 1, 1)))
    z[:, rng.integers(0, nh)] *= 40.0  # one loud head
    z = z.reshape(rows, nh * DH)
    z[7] = 0.0
    z16 = z.astype(np.float16)
    say(f"n_heads={nh} clip={clip} rows={rows}")
    zr = torch.empty((rows, nh * DH), dtype=torch.float32, device="cuda")
    q, s = qr.cross_head_had_quant(dev(z16), nh, clip, z_rot_out=zr)
    err, f = check(z16, nh, clip, host(q), host(s), host(zr))
    say(f"  rotated values max row-relative error {err:.2e}, code diff frac {f:.2e}")
    assert float(host(s)[7]) == float(np.float16(clip * 1e-5 / 7))
    assert not host(q)[7].any()


def test_cross_head_strided_rows():
    """ld_z > d and ld_q > d/2: the kernel reads only the first d elements of
    each input row and writes only the first d/2 bytes of each code row."""
    nh, rows = 16, 37
    d = nh * DH
    rng = np.random.default_rng(5)
    big = (rng.standard_normal((rows, d + 24)) * 3.0).astype(np.float16)
    z_dev = dev(big)[:, :d]
    q_full = torch.full((rows, d // 2 + 48), 0xA5, dtype=torch.uint8, device="cuda")
    q_view = q_full[:, : d // 2]
    s = torch.empty((rows,), dtype=torch.float16, device="cuda")
    zr = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    say(f"strided: rows={rows} ld_z={d + 24} ld_q={d // 2 + 48}")
    qr.cross_head_had_quant(z_dev, nh, 1.0, q_out=q_view, scale_out=s, z_rot_out=zr)
    qf = host(q_full)
    assert np.all(qf[:, d // 2:] == 0xA5)
    check(np.ascontiguousarray(big[:, :d]), nh, 1.0, qf[:, : d // 2], host(s), host(zr))


@pytest.mark.parametrize("nh", [4, 32])
def test_cross_head_unaligned_rows(nh):
    """ld_z % 8 != 0 (4-byte aligned rows) and an odd ld_q, with clip 0.9: the
    kernel reads only the first d elements of each row and writes only the
    first d/2 bytes of each code row."""
    rows = 29
    d = nh * DH
    rng = np.random.default_rng(11 + nh)
    big = (rng.standard_normal((rows, d + 2)) * 2.0).astype(np.float16)
    z_dev = dev(big)[:, :d]
    q_full = torch.full((rows, d // 2 + 1), 0x5A, dtype=torch.uint8, device="cuda")
    q_view = q_full[:, : d // 2]
    s = torch.empty((rows,), dtype=torch.float16, device="cuda")
    zr = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    say(f"unaligned: n_heads={nh} rows={rows} ld_z={d + 2} ld_q={d // 2 + 1}")
    qr.cross_head_had_quant(z_dev, nh, 0.9, q_out=q_view, scale_out=s, z_rot_out=zr)
    qf = host(q_full)
    assert np.all(qf[:, d // 2:] == 0x5A)
    check(np.ascontiguousarray(big[:, :d]), nh, 0.9, qf[:, : d // 2], host(s), host(zr))


def test_cross_head_no_rows():
    z = torch.empty((0, 4 * DH), dtype=torch.float16, device="cuda")
    q, s = qr.cross_head_had_quant(z, 4)
    torch.cuda.synchronize()
    assert q.shape == (0, 2 * DH) and s.shape == (0,)


@pytest.mark.parametrize("name,tokens", [("attn_out_7b", 512), ("attn_out_70b", 256)])
def test_cross_head_workload_rows(name, tokens):
    cfg = workloads.CROSS_HEAD_CONFIGS[name]
    z16 = workloads.make_attn_output(cfg, tokens=tokens)["z"]
    say(f"{name}: {tokens} x {cfg.d}")
    zr = torch.empty((tokens, cfg.d), dtype=torch.float32, device="cuda")
    q, s = qr.cross_head_had_quant(dev(z16), cfg.heads, z_rot_out=zr)
    err, f = check(z16, cfg.heads, 1.0, host(q), host(s), host(zr))
    say(f"  rotated values max row-relative error {err:.2e}, code diff frac {f:.2e}")


@pytest.mark.parametrize("name", ["attn_out_7b", "attn_out_70b"])
def test_cross_head_full_launch_sampled(name):
    """The whole workload in one launch (as timed, no z~ output); 64 sampled
    rows are checked against the oracle."""
    cfg = workloads.CROSS_HEAD_CONFIGS[name]
    z16 = workloads.make_attn_output(cfg)["z"]
    say(f"{name}: full launch {cfg.tokens} x {cfg.d}")
    q, s = qr.cross_head_had_quant(dev(z16), cfg.heads)
    qh, sh = host(q), host(s)
    rows = np.sort(np.random.default_rng(11).choice(cfg.tokens, 64, replace=False))
    rows[-1] = cfg.tokens - 1
    ref = oracle.cross_head_quant(z16[rows], cfg.heads)
    _, f = check_quant(oracle.unpack_int4(qh[rows]), sh[rows], ref["x_rot"], ref["scales"])
    say(f"  sampled code diff frac {f:.2e}")
