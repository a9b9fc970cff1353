"""The Python binding rejects tensors that do not match the layout the C entry points assume.

The C ABI takes raw pointers and sizes, so a wrong dtype, a transposed view, a short
buffer or a host tensor would reach the kernels unnoticed (wrong results or an access
past the allocation).  The binding checks every tensor first; these tests show each
check firing before any device entry point of the library is called (the device entry
points are replaced by a stub that fails the test if reached).  CPU only: host tensors
of the right layout are rejected for their device, after every other check passed.
"""

import os

import pytest
import torch

import recurrent_state_amd as rs

pytestmark = pytest.mark.skipif(not os.path.exists(rs.LIB_PATH), reason="library not built")

DEVICE_CALLS = ("taylor_state_init", "taylor_attn_prefill", "taylor_attn_prefill_into", "taylor_attn_prefill_varlen",
                "taylor_attn_prefill_varlen_into", "taylor_attn_prefill_backward", "taylor_attn_decode_step")


class _NoDeviceCalls:
    """The loaded library with its device entry points replaced by a stub that fails the test."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in DEVICE_CALLS:
            def stub(*args):
                raise AssertionError(f"{name} reached the library")
            return stub
        return getattr(self._real, name)


@pytest.fixture
def guarded(monkeypatch):
    real = rs.lib()
    monkeypatch.setattr(rs, "lib", lambda: _NoDeviceCalls(real))
    return rs


def _qkv(B=2, H=3, N=40, dk=16, dv=64, dtype=torch.float32):
    g = torch.Generator().manual_seed(0)
    return (torch.randn((B, H, N, dk), generator=g).to(dtype), torch.randn((B, H, N, dk), generator=g).to(dtype),
            torch.randn((B, H, N, dv), generator=g).to(dtype))


def test_prefill_checks_dtype_shape_contiguity_and_device(guarded):
    cfg = rs.config(3, 16, 64, 64, 1.0, rs.TAYLOR_F32)
    B, H, N = 2, 3, 40
    q, k, v = _qkv(B, H, N)
    o = torch.empty((B, H, N, 64))
    st = torch.zeros((B, H, rs.taylor_state_stride(cfg)))
    ws = torch.empty((max(16, rs.taylor_prefill_workspace_bytes(cfg, B, H, N)),), dtype=torch.uint8)
    # bfloat16 tensors under a float32 config
    with pytest.raises(TypeError, match="dtype"):
        rs.taylor_attn_prefill(q.bfloat16(), k, v, o, st, ws, cfg)
    with pytest.raises(TypeError, match="dtype"):
        rs.taylor_attn_prefill(q, k, v, o.double(), st, ws, cfg)
    # a [B, N, H, d] tensor viewed as [B, H, N, d]: right shape, wrong strides
    qt = q.transpose(1, 2).contiguous().transpose(1, 2)
    assert qt.shape == q.shape and not qt.is_contiguous()
    with pytest.raises(ValueError, match="contiguous"):
        rs.taylor_attn_prefill(qt, k, v, o, st, ws, cfg)
    # short last dimensions of v, o and the state
    with pytest.raises(ValueError, match="shape"):
        rs.taylor_attn_prefill(q, k, v[..., :32].contiguous(), o, st, ws, cfg)
    with pytest.raises(ValueError, match="shape"):
        rs.taylor_attn_prefill(q, k, v, o[..., :60].contiguous(), st, ws, cfg)
    with pytest.raises(ValueError, match="shape"):
        rs.taylor_attn_prefill(q, k, v, o, st[..., :100].contiguous(), ws, cfg)
    # k whose head width is not cfg.d_k, and q of another length than k
    with pytest.raises(ValueError, match="shape"):
        rs.taylor_attn_prefill(q, k[..., :8].contiguous(), v, o, st, ws, cfg)
    with pytest.raises(ValueError, match="shape"):
        rs.taylor_attn_prefill(q[:, :, :20].contiguous(), k, v, o, st, ws, cfg)
    # a workspace smaller than the library asks for
    need = rs.taylor_prefill_workspace_bytes(cfg, B, H, N)
    if need > 0:
        with pytest.raises(ValueError, match="workspace"):
            rs.taylor_attn_prefill(q, k, v, o, st, ws[: need - 1], cfg)
    # everything right but on the host
    with pytest.raises(ValueError, match="cuda"):
        rs.taylor_attn_prefill(q, k, v, o, st, ws, cfg)
    with pytest.raises(ValueError, match="cuda"):
        rs.taylor_attn_prefill_into(q, k, v, o, None, st, ws, cfg)


def test_prefill_into_checks_both_states(guarded):
    cfg = rs.config(3, 16, 64, 64, 1.0, rs.TAYLOR_BF16)
    B, H, N = 1, 2, 70
    q, k, v = _qkv(B, H, N, dtype=torch.bfloat16)
    stride = rs.taylor_state_stride(cfg)
    good = torch.zeros((B, H, stride))
    ws = torch.empty((max(16, rs.taylor_prefill_workspace_bytes(cfg, B, H, N)),), dtype=torch.uint8)
    with pytest.raises(ValueError, match="state_in"):
        rs.taylor_attn_prefill_into(q, k, v, None, torch.zeros((B, H, stride - 4)), good, ws, cfg)
    with pytest.raises(TypeError, match="state_out"):
        rs.taylor_attn_prefill_into(q, k, v, None, good, torch.zeros((B, H, stride), dtype=torch.float64), ws, cfg)
    with pytest.raises(TypeError, match="dtype"):
        rs.taylor_attn_prefill_into(q.float(), k, v, None, None, good, ws, cfg)


def test_varlen_checks_cu_seqlens_and_packing(guarded):
    cfg = rs.config(3, 16, 64, 64, 1.0, rs.TAYLOR_F32)
    H, T = 2, 100
    g = torch.Generator().manual_seed(1)
    q, k = torch.randn((H, T, 16), generator=g), torch.randn((H, T, 16), generator=g)
    v, o = torch.randn((H, T, 64), generator=g), torch.empty((H, T, 64))
    cu = torch.tensor([0, 30, 100], dtype=torch.int32)
    st = torch.zeros((2, H, rs.taylor_state_stride(cfg)))
    ws = torch.empty((max(16, rs.taylor_prefill_varlen_workspace_bytes(cfg, 2, H, 70, T)),), dtype=torch.uint8)
    with pytest.raises(TypeError, match="cu_seqlens"):
        rs.taylor_attn_prefill_varlen(q, k, v, o, st, ws, cu.long(), 70, cfg)
    with pytest.raises(ValueError, match="contiguous"):
        rs.taylor_attn_prefill_varlen(q, k, v, o, st, ws, torch.tensor([0, 0, 30, 0, 100], dtype=torch.int32)[::2],
                                      70, cfg)
    with pytest.raises(ValueError, match="shape"):
        rs.taylor_attn_prefill_varlen(q, k, v, o, st[:1].contiguous(), ws, cu, 70, cfg)
    with pytest.raises(ValueError, match="shape"):  # [T, H, d] packing instead of [H, T, d]
        rs.taylor_attn_prefill_varlen(q.transpose(0, 1).contiguous(), k, v, o, st, ws, cu, 70, cfg)
    with pytest.raises(ValueError, match="cuda"):
        rs.taylor_attn_prefill_varlen_into(q, k, v, o, None, st, ws, cu, 70, cfg)


def test_decode_and_state_init_checks(guarded):
    cfg = rs.config(3, 16, 64, 64, 1.0, rs.TAYLOR_F32)
    B, H = 4, 2
    q, k, v = (t[:, :, 0].contiguous() for t in _qkv(B, H, 1))
    o = torch.empty((B, H, 64))
    st = torch.zeros((B, H, rs.taylor_state_stride(cfg)))
    with pytest.raises(TypeError, match="dtype"):
        rs.taylor_attn_decode_step(q, k, v.bfloat16(), o, st, cfg)
    with pytest.raises(ValueError, match="shape"):
        rs.taylor_attn_decode_step(q, k, v, o, st[:, :, :9945].contiguous(), cfg)
    with pytest.raises(ValueError, match="shape"):  # a prefill-shaped [B, H, 1, d] query
        rs.taylor_attn_decode_step(q[:, :, None], k, v, o, st, cfg)
    with pytest.raises(ValueError, match="cuda"):
        rs.taylor_attn_decode_step(q, k, v, o, st, cfg)
    with pytest.raises(ValueError, match="shape"):
        rs.taylor_state_init(torch.zeros((B, H, 100)), cfg)
    with pytest.raises(ValueError, match="cuda"):
        rs.taylor_state_init(st, cfg)


def test_backward_checks_every_gradient_buffer(guarded):
    cfg = rs.config(3, 16, 64, 64, 1.0, rs.TAYLOR_F32)
    B, H, N = 1, 2, 50
    q, k, v = _qkv(B, H, N)
    o, g = torch.empty((B, H, N, 64)), torch.empty((B, H, N, 64))
    dq, dk, dv = torch.empty((B, H, N, 16)), torch.empty((B, H, N, 16)), torch.empty((B, H, N, 64))
    ws = torch.empty((max(16, rs.taylor_prefill_backward_workspace_bytes(cfg, B, H, N)),), dtype=torch.uint8)
    with pytest.raises(TypeError, match="g has dtype"):
        rs.taylor_attn_prefill_backward(q, k, v, o, g.bfloat16(), None, None, dq, dk, dv, ws, cfg)
    with pytest.raises(ValueError, match="dv has shape"):
        rs.taylor_attn_prefill_backward(q, k, v, o, g, None, None, dq, dk, dv[..., :16].contiguous(), ws, cfg)
    with pytest.raises(ValueError, match="dstate"):
        rs.taylor_attn_prefill_backward(q, k, v, o, g, None, torch.zeros((B, H, 8)), dq, dk, dv, ws, cfg)
    with pytest.raises(ValueError, match="cuda"):
        rs.taylor_attn_prefill_backward(q, k, v, o, g, None, None, dq, dk, dv, ws, cfg)
