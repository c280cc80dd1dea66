"""Host-side argument checks of the Python binding (no GPU needed).

The binding passes raw pointers to the C ABI, which cannot see tensor sizes,
so undersized or non-contiguous buffers must be refused in Python before any
library call.  Here the device check of ``_need`` is relaxed so CPU tensors
stand in for device tensors, and every library entry point is replaced by a
trap: a case passes only if it raises ValueError before reaching the library.
"""

import pytest

torch = pytest.importorskip("torch")

import rotated_w4a4_amd._lib as L  # noqa: E402


class _Trap:
    def __getattr__(self, name):
        raise AssertionError(f"library call {name} reached")


@pytest.fixture()
def host_tensors(monkeypatch):
    def need(t, dtype, name, ndim=None):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if ndim is not None and t.dim() != ndim:
            raise ValueError(f"{name} must have {ndim} dims")

    monkeypatch.setattr(L, "_need", need)
    monkeypatch.setattr(L, "lib", lambda: _Trap())
    monkeypatch.setattr(L, "_stream", lambda s: None)


def _decode_args(B=2, Hq=8, Hkv=2, S=64, D=128):
    u8, f16 = torch.uint8, torch.float16
    return dict(q=torch.zeros((B, Hq, D), dtype=f16), signs=torch.ones(D, dtype=torch.int8),
                k_cache=torch.zeros((B, Hkv, S, D // 2), dtype=u8),
                k_scale=torch.zeros((B, Hkv, S), dtype=f16),
                v_cache=torch.zeros((B, Hkv, S, D // 2), dtype=u8),
                v_scale=torch.zeros((B, Hkv, S), dtype=f16), max_len=S)


@pytest.mark.parametrize("change", [
    dict(signs=torch.ones(100, dtype=torch.int8)),                       # short signs
    dict(signs=torch.ones(128, dtype=torch.int8), signs_stride_h=128),   # per head: needs 256
    dict(signs=torch.ones(512, dtype=torch.int8)[::2]),                  # not contiguous
    dict(out=torch.zeros((2, 8, 64), dtype=torch.float16)),              # wrong shape
    dict(out=torch.zeros((2, 128, 8), dtype=torch.float16).transpose(1, 2)),  # not contiguous
    dict(out_f32=torch.zeros((2, 4, 128), dtype=torch.float32)),         # wrong shape
    dict(signs_stride_h=-1),
])
def test_decode_refuses_undersized_buffers(host_tensors, change):
    a = _decode_args()
    a.update(change)
    with pytest.raises(ValueError):
        L.kv_decode_attention(**a)


def _kv_args(B=2, H=3, S=5, D=128, S_cache=8):
    f16 = torch.float16
    return dict(k=torch.zeros((B, H, S, D), dtype=f16), v=torch.zeros((B, H, S, D), dtype=f16),
                signs=torch.ones(D, dtype=torch.int8),
                k_cache=torch.zeros((B, H, S_cache, D // 2), dtype=torch.uint8),
                k_scale=torch.zeros((B, H, S_cache), dtype=f16),
                v_cache=torch.zeros((B, H, S_cache, D // 2), dtype=torch.uint8),
                v_scale=torch.zeros((B, H, S_cache), dtype=f16))


@pytest.mark.parametrize("change", [
    dict(signs=torch.ones(64, dtype=torch.int8)),
    dict(signs=torch.ones(128, dtype=torch.int8), signs_stride_h=128),   # 3 heads need 384
    dict(k_rot_out=torch.zeros((2, 3, 5, 64), dtype=torch.float32)),
    dict(v_rot_out=torch.zeros((2, 3, 4, 128), dtype=torch.float32)),
])
def test_kv_refuses_undersized_buffers(host_tensors, change):
    a = _kv_args()
    a.update(change)
    with pytest.raises(ValueError):
        L.kv_had_quant(**a)


@pytest.mark.parametrize("change", [
    dict(q_out=torch.zeros((4, 100), dtype=torch.uint8)),       # narrower than d/2
    dict(q_out=torch.zeros((5, 128), dtype=torch.uint8)),       # wrong row count
    dict(scale_out=torch.zeros(8, dtype=torch.float16)[::2]),   # not contiguous
    dict(signs=torch.ones(255, dtype=torch.int8)),
    dict(x_rot_out=torch.zeros((4, 255), dtype=torch.float32)),
])
def test_had_quant_refuses_undersized_buffers(host_tensors, change):
    a = dict(x=torch.zeros((4, 256), dtype=torch.float16))
    a.update(change)
    with pytest.raises(ValueError):
        L.had_quant(**a)


def test_had_m_shape_and_device(host_tensors):
    x = torch.zeros((4, 12288), dtype=torch.float16)
    with pytest.raises(ValueError):
        L.had_quant(x, m=12, had_m=torch.ones((12, 11), dtype=torch.int8))
    with pytest.raises(ValueError):
        L.had_quant(torch.zeros((4, 256), dtype=torch.float16), m=1,
                    had_m=torch.ones((1, 1), dtype=torch.int8))


def test_swiglu_up_must_match_gate(host_tensors):
    g = torch.zeros((4, 256), dtype=torch.float16)
    with pytest.raises(ValueError):
        L.swiglu_had_quant(g, torch.zeros((4, 128), dtype=torch.float16))
