"""GPU parity of rotate+quant with the caller's small Hadamard factor H_m.

"QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (paper-graph-ui
summary), section 3.4 Stage 1a: for d = 2^n m the rotation is
H_{2^n} (x) H_m with any known Hadamard matrix H_m.  The library takes H_m
as data (``had_m``); these cases feed matrices other than the library's own
Paley ones -- rows and columns permuted and sign-flipped, a Kronecker
product, other orders -- and compare with the oracle given the same matrix.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from parity import check_quant, check_rot

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotated_w4a4_amd as qr  # noqa: E402


def say(msg: str) -> None:
    print(f"[had_m] {msg}", flush=True)


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def transformed(h: np.ndarray, seed: int) -> np.ndarray:
    """Rows and columns permuted and sign-flipped: still Hadamard."""
    rng = np.random.default_rng(seed)
    m = h.shape[0]
    h = h[rng.permutation(m)][:, rng.permutation(m)]
    return (h * (1 - 2 * rng.integers(0, 2, m))[:, None]
            * (1 - 2 * rng.integers(0, 2, m))[None, :]).astype(np.int8)


def factor(m: int, seed: int) -> np.ndarray:
    if m == 16:  # no Paley I of order 16: the Kronecker square of Paley H_4
        h4 = oracle.hadamard_m(4).astype(np.int64)
        return transformed(np.kron(h4, h4).astype(np.int8), seed)
    return transformed(oracle.hadamard_m(m), seed)


def run(d, m, hm, rows, seed, clip=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, d)).astype(np.float32)
    x[:, rng.integers(0, d, 3)] *= 60.0
    x16 = x.astype(np.float16)
    signs = (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)
    xr = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    q, s = qr.had_quant(dev(x16), dev(signs), m, clip, x_rot_out=xr, had_m=hm)
    ref = oracle.had_quant(x16, signs, m, clip, hm)
    e = check_rot(host(xr), ref["x_rot"])
    ns, f = check_quant(oracle.unpack_int4(host(q)), host(s), ref["x_rot"], ref["scales"])
    return e, ns, f


@pytest.mark.parametrize("m,rows", [(12, 600), (28, 300)])
def test_kronecker_kernel_with_another_factor(m, rows):
    hm = factor(m, 100 + m)
    assert not np.array_equal(hm, oracle.hadamard_m(m))
    say(f"kron d={1024 * m} m={m} rows={rows}, permuted/sign-flipped Paley")
    e, ns, f = run(1024 * m, m, hm, rows, m)
    say(f"  rot err {e:.2e}, scale ulps {ns}, code diff frac {f:.2e}")


@pytest.mark.parametrize("d,m", [(1024, 4), (1024, 8), (1024, 16), (1280, 20), (3072, 24),
                                 (32768, 32), (4096, 4), (8192, 8), (640, 20), (1536, 12),
                                 (896, 28)])
def test_generic_kernel_other_orders(d, m):
    hm = factor(m, d + m)
    say(f"generic d={d} m={m}")
    e, ns, f = run(d, m, hm, 23, d + m, clip=0.9 if m == 20 else 1.0)
    say(f"  rot err {e:.2e}, scale ulps {ns}, code diff frac {f:.2e}")


def test_library_factor_equals_default():
    # passing the library's own Paley matrix explicitly gives the same bytes
    rng = np.random.default_rng(5)
    x16 = rng.standard_normal((64, 12288)).astype(np.float16)
    signs = dev((1 - 2 * rng.integers(0, 2, 12288)).astype(np.int8))
    q1, s1 = qr.had_quant(dev(x16), signs, 12)
    q2, s2 = qr.had_quant(dev(x16), signs, 12, had_m=qr.hadamard_factor(12))
    np.testing.assert_array_equal(host(q1), host(q2))
    np.testing.assert_array_equal(host(s1), host(s2))
