"""ctypes binding of libquarot (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libquarot.so")
_lib = None

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_f32 = ctypes.c_float

_SIGNATURES = {
    "quarot_had_quant": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _i32, _vp, _f32,
                                        _vp, _i64, _vp, _vp, _vp]),
    "quarot_swiglu_had_quant": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp,
                                               _f32, _vp, _i64, _vp, _vp, _vp]),
    "quarot_cross_head_had_quant": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i64, _f32, _vp, _i64,
                                                   _vp, _vp, _vp]),
    "quarot_w4a4_gemm": (ctypes.c_int, [_vp, _i64, _vp, _vp, _i64, _vp, _i64, _i64, _i64,
                                        _vp, _i64, _vp, _i64, _vp]),
    "quarot_kv_had_quant": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                           _vp, _i64, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp,
                                           _i64, _i64, _vp, _vp, _vp]),
    "quarot_kv_decode_attention": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _i32,
                                                  _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp,
                                                  _f32, _i32, _vp, _vp, _vp, _i64, _vp]),
    "quarot_kv_decode_attention_noalloc": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i64, _vp, _i64,
                                                          _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                                          _i64, _i64, _vp, _f32, _i32, _vp, _vp,
                                                          _vp]),
    "quarot_kv_decode_workspace_bytes": (ctypes.c_int64, [_i64, _i64, _i64, _i64, _i64]),
    "quarot_hadamard_factor": (ctypes.c_int, [_i32, _vp]),
    "quarot_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "quarot_last_error": (ctypes.c_char_p, []),
}


class QuarotError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status
        self.detail = detail


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libquarot.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m rotated_w4a4_amd.build` "
                "(there is no fallback implementation)")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        detail = lib().quarot_last_error().decode(errors="replace")
        raise QuarotError(fn, status, detail)


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t, dtype, name: str, ndim: Optional[int] = None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def hadamard_factor(m: int) -> np.ndarray:
    """One of the library's Paley Hadamard matrices (int8 [m, m], +-1; m = 1, 12, 28)."""
    out = np.zeros((m, m), dtype=np.int8)
    _check("quarot_hadamard_factor",
           lib().quarot_hadamard_factor(m, out.ctypes.data_as(ctypes.c_void_p)))
    return out


def _had_m_host(m: int, had_m):
    """The host int8 [m, m] array passed as had_m (None for m = 1).  Without
    an explicit matrix the library's own Paley matrix of order m is used."""
    if m == 1:
        if had_m is not None:
            raise ValueError("had_m must be None when m = 1")
        return None
    if had_m is None:
        return hadamard_factor(m)
    if hasattr(had_m, "is_cuda"):
        if had_m.is_cuda:
            raise ValueError("had_m is read on the host: pass a CPU tensor or numpy array")
        had_m = had_m.numpy()
    h = np.ascontiguousarray(np.asarray(had_m), dtype=np.int8)
    if h.shape != (m, m):
        raise ValueError(f"had_m must be [{m}, {m}]")
    return h


def _host_ptr(a) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _had_quant_outputs(x, signs, q_out, scale_out, x_rot_out):
    torch = _torch()
    _need(x, torch.float16, "x", 2)
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    rows, d = x.shape
    if signs is not None:
        _need(signs, torch.int8, "signs", 1)
        if signs.numel() != d or not signs.is_contiguous():
            raise ValueError("signs must be a contiguous int8 vector of length d")
    if q_out is None:
        q_out = torch.empty((rows, d // 2), dtype=torch.uint8, device=x.device)
    if scale_out is None:
        scale_out = torch.empty((rows,), dtype=torch.float16, device=x.device)
    _need(q_out, torch.uint8, "q_out", 2)
    _need(scale_out, torch.float16, "scale_out", 1)
    if x_rot_out is not None:
        _need(x_rot_out, torch.float32, "x_rot_out", 2)
        if not x_rot_out.is_contiguous() or tuple(x_rot_out.shape) != (rows, d):
            raise ValueError("x_rot_out must be contiguous float32 [rows, d]")
    if q_out.stride(1) != 1 or q_out.shape[0] != rows or q_out.shape[1] < d // 2:
        raise ValueError("q_out must be [rows, >= d/2] uint8 with contiguous rows")
    if scale_out.shape[0] != rows or not scale_out.is_contiguous():
        raise ValueError("scale_out must be a contiguous fp16 [rows]")
    return rows, d, q_out, scale_out


def had_quant(x, signs=None, m: int = 1, clip_ratio: float = 1.0, q_out=None, scale_out=None,
              x_rot_out=None, had_m=None, stream=None):
    """Rotate+quant rows of fp16 x [rows, d] with H_{d/m} (x) H_m; returns
    (codes, scales).  had_m: int8 [m, m] host matrix (default: the library's
    Paley matrix of order m)."""
    rows, d, q_out, scale_out = _had_quant_outputs(x, signs, q_out, scale_out, x_rot_out)
    h = _had_m_host(m, had_m)
    st = lib().quarot_had_quant(_ptr(x), rows, d, x.stride(0), _ptr(signs), m, _host_ptr(h),
                                float(clip_ratio), _ptr(q_out), q_out.stride(0),
                                _ptr(scale_out), _ptr(x_rot_out), _stream(stream))
    _check("quarot_had_quant", st)
    return q_out, scale_out


def swiglu_had_quant(gate, up, signs=None, m: int = 1, clip_ratio: float = 1.0, q_out=None,
                     scale_out=None, x_rot_out=None, had_m=None, stream=None):
    """Rotate+quant of the gated product SiLU(gate) * up, rows of fp16
    [rows, d] each, formed in the same pass; returns (codes, scales)."""
    torch = _torch()
    rows, d, q_out, scale_out = _had_quant_outputs(gate, signs, q_out, scale_out, x_rot_out)
    _need(up, torch.float16, "up", 2)
    if tuple(up.shape) != (rows, d) or up.stride(1) != 1:
        raise ValueError("up must be [rows, d] with contiguous rows, like gate")
    h = _had_m_host(m, had_m)
    st = lib().quarot_swiglu_had_quant(_ptr(gate), _ptr(up), rows, d, gate.stride(0),
                                       up.stride(0), _ptr(signs), m, _host_ptr(h),
                                       float(clip_ratio), _ptr(q_out), q_out.stride(0),
                                       _ptr(scale_out), _ptr(x_rot_out), _stream(stream))
    _check("quarot_swiglu_had_quant", st)
    return q_out, scale_out


def cross_head_had_quant(z, n_heads: int, clip_ratio: float = 1.0, q_out=None, scale_out=None,
                         z_rot_out=None, stream=None):
    """Cross-head transform (H_{n_heads} over the head index, normalised) then
    per-token INT4 of rows of fp16 z [rows, n_heads * 128]; returns (codes, scales)."""
    rows, d, q_out, scale_out = _had_quant_outputs(z, None, q_out, scale_out, z_rot_out)
    if n_heads <= 0 or d % n_heads:
        raise ValueError("n_heads must divide the row length")
    st = lib().quarot_cross_head_had_quant(_ptr(z), rows, int(n_heads), d // int(n_heads),
                                           z.stride(0), float(clip_ratio), _ptr(q_out),
                                           q_out.stride(0), _ptr(scale_out), _ptr(z_rot_out),
                                           _stream(stream))
    _check("quarot_cross_head_had_quant", st)
    return q_out, scale_out


def w4a4_gemm(a_q, a_scale, b_q, b_scale, k: int, out=None, acc_out=None, stream=None):
    """fp16 [M, N] = dequant(int4 a_q [M, k/2] x int4 b_q [N, k/2]^T)."""
    torch = _torch()
    _need(a_q, torch.uint8, "a_q", 2)
    _need(b_q, torch.uint8, "b_q", 2)
    _need(a_scale, torch.float16, "a_scale", 1)
    _need(b_scale, torch.float16, "b_scale", 1)
    if a_q.stride(1) != 1 or b_q.stride(1) != 1:
        raise ValueError("a_q/b_q rows must be contiguous")
    M, N = a_q.shape[0], b_q.shape[0]
    if a_scale.numel() != M or b_scale.numel() != N:
        raise ValueError("scale lengths must match M and N")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=a_q.device)
    _need(out, torch.float16, "out", 2)
    if out.stride(1) != 1 or tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N] with contiguous rows")
    ld_acc = 0
    if acc_out is not None:
        _need(acc_out, torch.int32, "acc_out", 2)
        if acc_out.stride(1) != 1 or tuple(acc_out.shape) != (M, N):
            raise ValueError("acc_out must be [M, N] with contiguous rows")
        ld_acc = acc_out.stride(0)
    st = lib().quarot_w4a4_gemm(_ptr(a_q), a_q.stride(0), _ptr(a_scale), _ptr(b_q),
                                b_q.stride(0), _ptr(b_scale), M, N, int(k), _ptr(out),
                                out.stride(0), _ptr(acc_out), ld_acc, _stream(stream))
    _check("quarot_w4a4_gemm", st)
    return out


def _check_signs(signs, length: int, name: str = "signs") -> None:
    """signs: a contiguous int8 device vector of at least `length` entries."""
    torch = _torch()
    if signs is None:
        return
    _need(signs, torch.int8, name)
    if not signs.is_contiguous() or signs.numel() < length:
        raise ValueError(f"{name} must be a contiguous int8 tensor of at least {length} entries")


def kv_had_quant(k, v, signs, k_cache, k_scale, v_cache=None, v_scale=None, pos0: int = 0,
                 signs_stride_h: int = 0, clip_ratio: float = 1.0, mode: int = 0,
                 k_zero=None, v_zero=None, k_rot_out=None, v_rot_out=None, stream=None):
    """Quantise K (and V) [B, H, S, D] into caches [B, H, S_cache, D/2] at pos0.

    mode 0: symmetric int4 codes + fp16 scales.  mode 1: asymmetric uint4
    codes + fp16 scales + fp16 zero points (k_zero / v_zero, shaped like the
    scales); the pages use clip_ratio 0.95 for it.  k_rot_out / v_rot_out:
    optional float32 [B, H, S, D] receiving the rotated groups."""
    torch = _torch()
    ref = k if k is not None else v
    _need(ref, torch.float16, "k/v", 4)
    B, H, S, D = ref.shape
    for name, t in (("k", k), ("v", v)):
        if t is None:
            continue
        _need(t, torch.float16, name, 4)
        if tuple(t.shape) != (B, H, S, D) or t.stride(3) != 1:
            raise ValueError(f"{name} must be [B, H, S, D] with contiguous D")
        if t.stride() != ref.stride():
            raise ValueError("k and v must share strides")
    caches = [(k, k_cache, k_scale, k_zero, "k"), (v, v_cache, v_scale, v_zero, "v")]
    S_cache = None
    for t, cq, cs, cz, name in caches:
        if t is None:
            continue
        if mode == 1:
            _need(cz, torch.float16, f"{name}_zero", 3)
            if not cz.is_contiguous() or tuple(cz.shape) != tuple(cs.shape):
                raise ValueError(f"{name}_zero must be contiguous and shaped like {name}_scale")
        _need(cq, torch.uint8, f"{name}_cache", 4)
        _need(cs, torch.float16, f"{name}_scale", 3)
        if not cq.is_contiguous() or not cs.is_contiguous():
            raise ValueError("caches must be contiguous")
        if cq.shape[0] != B or cq.shape[1] != H or cq.shape[3] != D // 2:
            raise ValueError(f"{name}_cache must be [B, H, S_cache, D/2]")
        if tuple(cs.shape) != tuple(cq.shape[:3]):
            raise ValueError(f"{name}_scale must be [B, H, S_cache]")
        if S_cache is None:
            S_cache = cq.shape[2]
        elif cq.shape[2] != S_cache:
            raise ValueError("k and v caches must have the same length")
    if signs_stride_h < 0:
        raise ValueError("signs_stride_h must be >= 0")
    _check_signs(signs, int(signs_stride_h) * (H - 1) + D)
    for name, t, r in (("k_rot_out", k, k_rot_out), ("v_rot_out", v, v_rot_out)):
        if r is None:
            continue
        if t is None:
            raise ValueError(f"{name} given without its tensor")
        _need(r, torch.float32, name, 4)
        if not r.is_contiguous() or tuple(r.shape) != (B, H, S, D):
            raise ValueError(f"{name} must be contiguous float32 [B, H, S, D]")
    sb, sh, ss, _ = ref.stride()
    st = lib().quarot_kv_had_quant(_ptr(k), _ptr(v), B, H, S, D, sb, sh, ss, _ptr(signs),
                                   int(signs_stride_h), int(mode), float(clip_ratio),
                                   _ptr(k_cache) if k is not None else None,
                                   _ptr(k_scale) if k is not None else None,
                                   _ptr(k_zero) if (k is not None and mode == 1) else None,
                                   _ptr(v_cache) if v is not None else None,
                                   _ptr(v_scale) if v is not None else None,
                                   _ptr(v_zero) if (v is not None and mode == 1) else None,
                                   S_cache, int(pos0), _ptr(k_rot_out), _ptr(v_rot_out),
                                   _stream(stream))
    _check("quarot_kv_had_quant", st)
    if mode == 1:
        return k_cache, k_scale, k_zero, v_cache, v_scale, v_zero
    return k_cache, k_scale, v_cache, v_scale


def kv_decode_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, max_len: int) -> int:
    """Workspace bytes kv_decode_attention needs for these sizes."""
    n = int(lib().quarot_kv_decode_workspace_bytes(B, Hq, Hkv, D, max_len))
    _check("quarot_kv_decode_workspace_bytes", n if n < 0 else 0)
    return n


def _decode_prepare(q, signs, k_cache, k_scale, v_cache, v_scale, lengths, mode, k_zero, v_zero,
                    sm_scale, signs_stride_h, out, out_f32):
    """Shared argument checks of the two decode calls; returns the sizes and
    the (possibly allocated) outputs."""
    torch = _torch()
    _need(q, torch.float16, "q", 3)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    B, Hq, D = q.shape
    _need(k_cache, torch.uint8, "k_cache", 4)
    _need(v_cache, torch.uint8, "v_cache", 4)
    _need(k_scale, torch.float16, "k_scale", 3)
    _need(v_scale, torch.float16, "v_scale", 3)
    Hkv, S_cache = k_cache.shape[1], k_cache.shape[2]
    for name, c, sc in (("k", k_cache, k_scale), ("v", v_cache, v_scale)):
        if not c.is_contiguous() or not sc.is_contiguous():
            raise ValueError(f"{name} cache buffers must be contiguous")
        if tuple(c.shape) != (B, Hkv, S_cache, D // 2) or tuple(sc.shape) != (B, Hkv, S_cache):
            raise ValueError(f"{name}_cache must be [B, Hkv, S_cache, D/2] with scales [B, Hkv, S_cache]")
    if mode == 1:
        for name, z in (("k_zero", k_zero), ("v_zero", v_zero)):
            _need(z, torch.float16, name, 3)
            if not z.is_contiguous() or tuple(z.shape) != (B, Hkv, S_cache):
                raise ValueError(f"{name} must be contiguous [B, Hkv, S_cache]")
    if signs_stride_h < 0:
        raise ValueError("signs_stride_h must be >= 0")
    _check_signs(signs, int(signs_stride_h) * (Hkv - 1) + D)
    if lengths is not None:
        _need(lengths, torch.int32, "lengths", 1)
        if lengths.shape[0] != B or not lengths.is_contiguous():
            raise ValueError("lengths must be a contiguous int32 [B]")
    if sm_scale is None:
        sm_scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=q.device)
    _need(out, torch.float16, "out", 3)
    if not out.is_contiguous() or tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be contiguous fp16 [B, Hq, D]")
    if out_f32 is not None:
        _need(out_f32, torch.float32, "out_f32", 3)
        if not out_f32.is_contiguous() or tuple(out_f32.shape) != (B, Hq, D):
            raise ValueError("out_f32 must be contiguous float32 [B, Hq, D]")
    return B, Hq, Hkv, D, S_cache, float(sm_scale), out


def kv_decode_attention(q, signs, k_cache, k_scale, v_cache, v_scale, max_len: int,
                        lengths=None, mode: int = 0, k_zero=None, v_zero=None,
                        sm_scale: Optional[float] = None, cross_head: bool = False,
                        signs_stride_h: int = 0, out=None, out_f32=None, workspace=None,
                        stream=None):
    """One decode step: q fp16 [B, Hq, 128] against the int4 caches
    [B, Hkv, S_cache, 64] (+ fp16 scales [B, Hkv, S_cache], and zero points in
    mode 1).  Returns fp16 [B, Hq, 128] (``out``); ``out_f32`` optionally
    receives an fp32 copy.  ``workspace`` (uint8, device) is allocated here
    when not given."""
    torch = _torch()
    B, Hq, Hkv, D, S_cache, sm_scale, out = _decode_prepare(
        q, signs, k_cache, k_scale, v_cache, v_scale, lengths, mode, k_zero, v_zero, sm_scale,
        signs_stride_h, out, out_f32)
    need = kv_decode_workspace_bytes(B, Hq, Hkv, D, max_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, torch.uint8, "workspace", 1)
    st = lib().quarot_kv_decode_attention(
        _ptr(q), B, Hq, Hkv, D, _ptr(signs), int(signs_stride_h), int(mode),
        _ptr(k_cache), _ptr(k_scale), _ptr(k_zero) if mode == 1 else None,
        _ptr(v_cache), _ptr(v_scale), _ptr(v_zero) if mode == 1 else None,
        S_cache, int(max_len), _ptr(lengths), sm_scale, int(bool(cross_head)),
        _ptr(out), _ptr(out_f32), _ptr(workspace), workspace.numel(), _stream(stream))
    _check("quarot_kv_decode_attention", st)
    return out


def kv_decode_attention_noalloc(q, signs, k_cache, k_scale, v_cache, v_scale, max_len: int,
                                lengths=None, mode: int = 0, k_zero=None, v_zero=None,
                                sm_scale: Optional[float] = None, cross_head: bool = False,
                                signs_stride_h: int = 0, out=None, out_f32=None, stream=None):
    """kv_decode_attention without a workspace: the partials go to the
    library's own scratch array (QUAROT_DECODE_SCRATCH_BYTES per GPU).  With
    ``out`` given, nothing is allocated."""
    B, Hq, Hkv, D, S_cache, sm_scale, out = _decode_prepare(
        q, signs, k_cache, k_scale, v_cache, v_scale, lengths, mode, k_zero, v_zero, sm_scale,
        signs_stride_h, out, out_f32)
    st = lib().quarot_kv_decode_attention_noalloc(
        _ptr(q), B, Hq, Hkv, D, _ptr(signs), int(signs_stride_h), int(mode),
        _ptr(k_cache), _ptr(k_scale), _ptr(k_zero) if mode == 1 else None,
        _ptr(v_cache), _ptr(v_scale), _ptr(v_zero) if mode == 1 else None,
        S_cache, int(max_len), _ptr(lengths), sm_scale, int(bool(cross_head)),
        _ptr(out), _ptr(out_f32), _stream(stream))
    _check("quarot_kv_decode_attention_noalloc", st)
    return out
