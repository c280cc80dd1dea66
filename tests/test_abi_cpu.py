"""Host-side checks of libquarot (no GPU needed).

* the library loads and exports every function declared in include/quarot.h;
* its Paley factors equal the oracle's (two independent constructions of
  the same published definition);
* the caller's H_m (host memory) is validated: +-1 entries, H H^T = m I;
* invalid arguments are rejected with the documented status before any HIP
  call (no call here reaches the device: each one fails validation).
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import rotated_w4a4_amd as qr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, MISALIGNED, HIPERR = 0, -1, -2, -3, -4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qr.library_path()):
        pytest.skip("libquarot.so not built")
    return qr.lib()


def test_exports_every_declared_symbol(lib):
    with open(os.path.join(ROOT, "include", "quarot.h")) as f:
        text = f.read()
    names = set(re.findall(r"\b(quarot_[a-z0-9_]+)\s*\(", text))
    assert {"quarot_had_quant", "quarot_w4a4_gemm", "quarot_kv_had_quant",
            "quarot_kv_decode_attention", "quarot_kv_decode_workspace_bytes",
            "quarot_swiglu_had_quant", "quarot_cross_head_had_quant",
            "quarot_kv_decode_attention_noalloc"} <= names
    assert "quarot_rmsnorm_had_quant" not in names
    for name in names:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("m", [1, 12, 28])
def test_builtin_factor_matches_oracle(lib, m):
    np.testing.assert_array_equal(qr.hadamard_factor(m), oracle.hadamard_m(m))


def test_factor_unsupported(lib):
    out = np.zeros(64, np.int8)
    assert lib.quarot_hadamard_factor(20, out.ctypes.data_as(ctypes.c_void_p)) == UNSUPPORTED
    assert lib.quarot_hadamard_factor(12, None) == INVALID


def test_status_strings(lib):
    for s in (OK, INVALID, UNSUPPORTED, MISALIGNED, HIPERR, 7):
        assert lib.quarot_status_string(s)


FAKE = 0x10000  # 64 KiB-aligned host address never dereferenced by a failing call


P12 = oracle.hadamard_m(12)


def _hq(lib, **kw):
    a = dict(x=FAKE, rows=4, d=256, ld_x=256, signs=None, m=1, had_m=None, clip=1.0, q=FAKE,
             ld_q=128, scale=FAKE, xrot=None, stream=None)
    a.update(kw)
    h = a["had_m"]
    hp = h.ctypes.data_as(ctypes.c_void_p) if isinstance(h, np.ndarray) else h
    return lib.quarot_had_quant(a["x"], a["rows"], a["d"], a["ld_x"], a["signs"], a["m"], hp,
                                a["clip"], a["q"], a["ld_q"], a["scale"], a["xrot"], a["stream"])


def _bad_entry():
    h = P12.copy()
    h[3, 5] = 0
    return h


def _not_orthogonal():
    h = P12.copy()
    h[3, 5] = -h[3, 5]  # +-1 entries, but rows 3 and 5 no longer orthogonal
    return h


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), INVALID),
    (dict(d=0), INVALID),
    (dict(clip=0.0), INVALID),
    (dict(clip=1.5), INVALID),
    (dict(clip=float("nan")), INVALID),
    (dict(m=20), INVALID),  # had_m missing
    (dict(m=5, had_m=np.ones((5, 5), np.int8)), UNSUPPORTED),
    (dict(m=36, had_m=np.ones((36, 36), np.int8)), UNSUPPORTED),
    (dict(m=2, had_m=np.ones((2, 2), np.int8)), UNSUPPORTED),
    (dict(m=1, had_m=np.ones((1, 1), np.int8)), INVALID),  # NULL iff m == 1
    (dict(m=12, d=12288, ld_x=12288, ld_q=6144), INVALID),  # had_m missing
    (dict(m=12, d=12288, ld_x=12288, ld_q=6144, had_m=_bad_entry()), INVALID),
    (dict(m=12, d=12288, ld_x=12288, ld_q=6144, had_m=_not_orthogonal()), INVALID),
    (dict(m=12, d=12288, ld_x=12288, ld_q=6144, had_m=np.ones((12, 12), np.int8)), INVALID),
    (dict(m=12, d=4096, ld_x=4096, ld_q=2048, had_m=P12), UNSUPPORTED),  # not 2^n * 12
    (dict(d=384, ld_x=384, ld_q=192), UNSUPPORTED),  # 384 = 3 * 128, not 2^n * 1
    (dict(d=48, m=12, had_m=P12, ld_x=48, ld_q=32), UNSUPPORTED),  # d % 32 != 0
    (dict(d=65536, ld_x=65536, ld_q=32768), UNSUPPORTED),
    (dict(ld_x=128), INVALID),
    (dict(ld_q=64), INVALID),
    (dict(x=None), INVALID),
    (dict(q=None), INVALID),
    (dict(scale=None), INVALID),
    (dict(x=FAKE + 8), MISALIGNED),
    (dict(ld_x=260), MISALIGNED),
    (dict(q=FAKE + 4), MISALIGNED),
    (dict(ld_q=136), MISALIGNED),
    (dict(scale=FAKE + 1), MISALIGNED),
    (dict(xrot=FAKE + 4), MISALIGNED),
])
def test_had_quant_rejects(lib, kw, status):
    assert _hq(lib, **kw) == status
    assert lib.quarot_last_error()


def test_had_m_check_reports_the_rows(lib):
    assert _hq(lib, m=12, d=12288, ld_x=12288, ld_q=6144, had_m=_not_orthogonal()) == INVALID
    assert b"not a Hadamard matrix" in lib.quarot_last_error()


def test_had_quant_zero_rows_is_noop(lib):
    assert _hq(lib, rows=0, x=None, q=None, scale=None) == OK


def _sw(lib, **kw):
    a = dict(g=FAKE, u=FAKE, rows=4, d=12288, ld_g=12288, ld_u=12288, signs=None, m=12,
             had_m=P12, clip=1.0, q=FAKE, ld_q=6144, s=FAKE, xr=None)
    a.update(kw)
    h = a["had_m"]
    hp = h.ctypes.data_as(ctypes.c_void_p) if isinstance(h, np.ndarray) else h
    return lib.quarot_swiglu_had_quant(a["g"], a["u"], a["rows"], a["d"], a["ld_g"], a["ld_u"],
                                       a["signs"], a["m"], hp, a["clip"], a["q"], a["ld_q"],
                                       a["s"], a["xr"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(u=None), INVALID),
    (dict(g=None), INVALID),
    (dict(ld_u=12000), INVALID),
    (dict(ld_u=12296 + 4), MISALIGNED),
    (dict(u=FAKE + 8), MISALIGNED),
    (dict(had_m=None), INVALID),
    (dict(had_m=_not_orthogonal()), INVALID),
    (dict(d=1000), UNSUPPORTED),
    (dict(clip=2.0), INVALID),
])
def test_swiglu_had_quant_rejects(lib, kw, status):
    assert _sw(lib, **kw) == status
    assert lib.quarot_last_error()


def test_swiglu_had_quant_zero_rows_is_noop(lib):
    assert _sw(lib, rows=0, g=None, u=None, q=None, s=None) == OK


def _gemm(lib, **kw):
    a = dict(a=FAKE, lda=64, sa=FAKE, b=FAKE, ldb=64, sb=FAKE, M=16, N=16, K=128, c=FAKE,
             ldc=16, acc=None, ld_acc=0)
    a.update(kw)
    return lib.quarot_w4a4_gemm(a["a"], a["lda"], a["sa"], a["b"], a["ldb"], a["sb"], a["M"],
                                a["N"], a["K"], a["c"], a["ldc"], a["acc"], a["ld_acc"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), INVALID),
    (dict(K=0), INVALID),
    (dict(K=48), UNSUPPORTED),
    (dict(K=65568, lda=32784, ldb=32784), UNSUPPORTED),
    (dict(lda=32), INVALID),
    (dict(ldc=8), INVALID),
    (dict(acc=FAKE, ld_acc=8), INVALID),
    (dict(a=None), INVALID),
    (dict(sb=None), INVALID),
    (dict(c=None), INVALID),
    (dict(a=FAKE + 8), MISALIGNED),
    (dict(lda=72), MISALIGNED),
    (dict(sa=FAKE + 1), MISALIGNED),
    (dict(c=FAKE + 1), MISALIGNED),
    (dict(acc=FAKE + 2, ld_acc=16), MISALIGNED),
    (dict(M=1 << 31), UNSUPPORTED),
    # 2^36 tiles of 256 x 256: more work items than a grid dimension holds;
    # rejected on the host before any launch
    (dict(M=(1 << 31) - 1, N=(1 << 31) - 1, ldc=(1 << 31) - 1), UNSUPPORTED),
])
def test_gemm_rejects(lib, kw, status):
    assert _gemm(lib, **kw) == status


def test_gemm_empty_is_noop(lib):
    assert _gemm(lib, M=0, a=None, c=None) == OK


def _kv(lib, **kw):
    a = dict(k=FAKE, v=FAKE, B=2, H=2, S=4, D=128, sb=1024, sh=512, ss=128, signs=None,
             ssh=0, mode=0, clip=1.0, kq=FAKE, ks=FAKE, kz=None, vq=FAKE, vs=FAKE, vz=None,
             S_cache=8, pos0=0, kr=None, vr=None)
    a.update(kw)
    return lib.quarot_kv_had_quant(a["k"], a["v"], a["B"], a["H"], a["S"], a["D"], a["sb"],
                                   a["sh"], a["ss"], a["signs"], a["ssh"], a["mode"], a["clip"],
                                   a["kq"], a["ks"], a["kz"], a["vq"], a["vs"], a["vz"],
                                   a["S_cache"], a["pos0"], a["kr"], a["vr"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INVALID),
    (dict(D=96), UNSUPPORTED),
    (dict(D=512), UNSUPPORTED),
    (dict(mode=2), INVALID),
    (dict(mode=1), INVALID),  # mode 1 needs the zero-point buffers
    (dict(mode=1, kz=FAKE), INVALID),
    (dict(mode=1, kz=FAKE, vz=FAKE + 1), MISALIGNED),
    (dict(clip=0.0), INVALID),
    (dict(pos0=5), INVALID),
    (dict(pos0=-1), INVALID),
    (dict(k=None, v=None), INVALID),
    (dict(kq=None), INVALID),
    (dict(vs=None), INVALID),
    (dict(ss=100), MISALIGNED),
    (dict(k=FAKE + 2), MISALIGNED),
    (dict(vq=FAKE + 4), MISALIGNED),
    (dict(ssh=-1), INVALID),
    (dict(kr=FAKE + 4), MISALIGNED),
    (dict(vr=FAKE + 8), MISALIGNED),
])
def test_kv_rejects(lib, kw, status):
    assert _kv(lib, **kw) == status


def test_kv_empty_is_noop(lib):
    assert _kv(lib, S=0, k=None) == OK


def _dec(lib, **kw):
    a = dict(q=FAKE, B=2, Hq=8, Hkv=2, D=128, signs=None, ssh=0, mode=0, kq=FAKE, ks=FAKE,
             kz=None, vq=FAKE, vs=FAKE, vz=None, S_cache=512, max_len=300, lengths=None,
             sm=0.088, cross=0, out=FAKE, out32=None, ws=FAKE, ws_bytes=1 << 20)
    a.update(kw)
    return lib.quarot_kv_decode_attention(a["q"], a["B"], a["Hq"], a["Hkv"], a["D"], a["signs"],
                                          a["ssh"], a["mode"], a["kq"], a["ks"], a["kz"], a["vq"],
                                          a["vs"], a["vz"], a["S_cache"], a["max_len"],
                                          a["lengths"], a["sm"], a["cross"], a["out"],
                                          a["out32"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INVALID),
    (dict(Hq=0), INVALID),
    (dict(Hq=6, Hkv=4), INVALID),
    (dict(D=64), UNSUPPORTED),
    (dict(Hq=32, Hkv=2), UNSUPPORTED),       # group of 16 query heads
    (dict(mode=2), INVALID),
    (dict(mode=1), INVALID),                 # zero points missing
    (dict(mode=1, kz=FAKE, vz=FAKE + 1), MISALIGNED),
    (dict(cross=2), INVALID),
    (dict(cross=1, Hq=6, Hkv=2), UNSUPPORTED),
    (dict(cross=1, Hq=512, Hkv=64), UNSUPPORTED),
    (dict(sm=0.0), INVALID),
    (dict(sm=float("inf")), INVALID),
    (dict(sm=float("nan")), INVALID),
    (dict(max_len=0), INVALID),
    (dict(max_len=513), INVALID),
    (dict(max_len=(1 << 24) + 1, S_cache=1 << 25), UNSUPPORTED),
    (dict(B=1 << 21, Hq=64, Hkv=8), UNSUPPORTED),  # 2^24 workgroups of 256 threads
    (dict(ssh=-1), INVALID),
    (dict(q=None), INVALID),
    (dict(vs=None), INVALID),
    (dict(out=None), INVALID),
    (dict(ws=None), INVALID),
    (dict(ws_bytes=64), INVALID),
    (dict(q=FAKE + 8), MISALIGNED),
    (dict(kq=FAKE + 4), MISALIGNED),
    (dict(ws=FAKE + 4), MISALIGNED),
    (dict(out=FAKE + 1), MISALIGNED),
    (dict(out32=FAKE + 2), MISALIGNED),
    (dict(lengths=FAKE + 2), MISALIGNED),
])
def test_decode_rejects(lib, kw, status):
    assert _dec(lib, **kw) == status


def _dec_na(lib, **kw):
    a = dict(q=FAKE, B=2, Hq=8, Hkv=2, D=128, signs=None, ssh=0, mode=0, kq=FAKE, ks=FAKE,
             kz=None, vq=FAKE, vs=FAKE, vz=None, S_cache=512, max_len=300, lengths=None,
             sm=0.088, cross=0, out=FAKE, o32=None)
    a.update(kw)
    return lib.quarot_kv_decode_attention_noalloc(
        a["q"], a["B"], a["Hq"], a["Hkv"], a["D"], a["signs"], a["ssh"], a["mode"], a["kq"],
        a["ks"], a["kz"], a["vq"], a["vs"], a["vz"], a["S_cache"], a["max_len"], a["lengths"],
        a["sm"], a["cross"], a["out"], a["o32"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=256, Hq=64, Hkv=8, S_cache=4096, max_len=4096), UNSUPPORTED),  # past the scratch
    (dict(D=64), UNSUPPORTED),
    (dict(mode=3), INVALID),
    (dict(q=None), INVALID),
    (dict(max_len=600), INVALID),
    (dict(q=FAKE + 8), MISALIGNED),
])
def test_decode_noalloc_rejects(lib, kw, status):
    assert _dec_na(lib, **kw) == status
    assert lib.quarot_last_error()


def test_decode_noalloc_scratch_limit_is_reported(lib):
    assert _dec_na(lib, B=256, Hq=64, Hkv=8, S_cache=4096, max_len=4096) == UNSUPPORTED
    assert b"allocation-free" in lib.quarot_last_error()
    assert _dec_na(lib, B=0) == OK


def test_decode_empty_batch_is_noop(lib):
    assert _dec(lib, B=0, q=None, out=None, ws=None) == OK


def test_decode_workspace_size(lib):
    # (B * Hkv * splits) slots per query head of the group, 130 floats each
    n = lib.quarot_kv_decode_workspace_bytes(16, 64, 8, 128, 4096)
    assert n > 0 and n % (130 * 4 * 8) == 0
    assert lib.quarot_kv_decode_workspace_bytes(1, 16, 1, 128, 100) == UNSUPPORTED
    assert lib.quarot_kv_decode_workspace_bytes(1, 8, 1, 128, 0) == INVALID
    sizes = [lib.quarot_kv_decode_workspace_bytes(2, 8, 2, 128, n) for n in range(1, 3000, 37)]
    assert all(s > 0 for s in sizes)


def _ch(lib, **kw):
    a = dict(z=FAKE, rows=4, nh=8, dh=128, ld_z=1024, clip=1.0, q=FAKE, ld_q=512, s=FAKE, zr=None)
    a.update(kw)
    return lib.quarot_cross_head_had_quant(a["z"], a["rows"], a["nh"], a["dh"], a["ld_z"],
                                           a["clip"], a["q"], a["ld_q"], a["s"], a["zr"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), INVALID),
    (dict(nh=0), INVALID),
    (dict(dh=0), INVALID),
    (dict(clip=0.0), INVALID),
    (dict(clip=float("nan")), INVALID),
    (dict(dh=64, ld_z=512, ld_q=256), UNSUPPORTED),
    (dict(nh=6, ld_z=768, ld_q=384), UNSUPPORTED),
    (dict(nh=128, ld_z=16384, ld_q=8192), UNSUPPORTED),
    (dict(ld_z=1000), INVALID),
    (dict(ld_q=500), INVALID),
    (dict(z=None), INVALID),
    (dict(q=None), INVALID),
    (dict(s=None), INVALID),
    (dict(z=FAKE + 2), MISALIGNED),
    (dict(ld_z=1025), MISALIGNED),
    (dict(s=FAKE + 1), MISALIGNED),
    (dict(zr=FAKE + 4), MISALIGNED),
])
def test_cross_head_had_quant_rejects(lib, kw, status):
    assert _ch(lib, **kw) == status
    assert lib.quarot_last_error()


def test_cross_head_had_quant_zero_rows_is_noop(lib):
    assert _ch(lib, rows=0, z=None, q=None, s=None) == OK
