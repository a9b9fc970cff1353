"""taylor_attn_prefill_into_static (the library's static per-GPU workspace, no allocation) against
taylor_attn_prefill_into with a caller-allocated workspace: the same kernels on the same inputs, so
the outputs and final states must agree bit for bit.  Two calls in a row, the second smaller (and a
third smaller still, continuing a state in place), each compared with the workspace form; the last is
also checked against the oracle at the float32 bar."""

import ctypes

import numpy as np
import pytest

import oracle
import recurrent_state_amd as rs
import synth
from gpu_util import TOL_BF16, announce, row_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(x, cfg, state_in=None, direct_abi=False):
    import torch

    q, k, v = x.torch(DEV)
    B, H, N = k.shape[:3]
    stride = rs.taylor_state_stride(cfg)
    o_ref = torch.empty((B, H, N, 64), device=DEV)
    st_ref = torch.empty((B, H, stride), device=DEV)
    rs.taylor_attn_prefill_into(q, k, v, o_ref, state_in, st_ref, rs.new_workspace(cfg, B, H, N, DEV), cfg)
    o = torch.full((B, H, N, 64), float("nan"), device=DEV)
    st = torch.full((B, H, stride), float("nan"), device=DEV)
    if direct_abi:
        rc = rs.lib().taylor_attn_prefill_into_static(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), None if state_in is None else state_in.data_ptr(),
            st.data_ptr(), B, H, N, ctypes.byref(cfg), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == rs.TAYLOR_OK, rs.taylor_status_string(rc)
    else:
        rs.taylor_attn_prefill_into_static(q, k, v, o, state_in, st, cfg)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), "outputs differ from the workspace form"
    assert torch.equal(st, st_ref), "final states differ from the workspace form"
    return o, st


def test_static_workspace_matches_the_workspace_form():
    import torch

    # 1: the bf16 benchmark shape (split form: state pass, scan, readout through the static array)
    announce("static-ws", "bf16 B4 H16 N8192")
    cfg = rs.config(3, 16, 64, 0, 1.0, rs.TAYLOR_BF16)
    assert rs.taylor_prefill_workspace_bytes(cfg, 4, 16, 8192) > 0
    _both(synth.make_qkv(3, 4, 16, 8192, 16, 64, synth.BF16), cfg, direct_abi=True)
    # 2: smaller, float32 feature-block kernel, continuing a nonzero incoming state
    announce("static-ws", "f32 B1 H8 N1000 from a state")
    cfg = rs.config(3, 16, 64, 0, 1.0, rs.TAYLOR_F32)
    x0 = synth.make_qkv(40, 1, 8, 700, 16, 64)
    st0 = torch.empty((1, 8, rs.taylor_state_stride(cfg)), device=DEV)
    rs.taylor_attn_prefill_into(*x0.torch(DEV), None, None, st0, rs.new_workspace(cfg, 1, 8, 700, DEV), cfg)
    _both(synth.make_qkv(41, 1, 8, 1000, 16, 64), cfg, state_in=st0, direct_abi=True)
    # 3: smaller still, bf16 n = 2, through the binding; the oracle on the whole sequence
    announce("static-ws", "bf16 n2 B2 H3 N300")
    cfg = rs.config(2, 16, 64, 0, 1.0, rs.TAYLOR_BF16)
    x = synth.make_qkv(42, 2, 3, 300, 16, 64, synth.BF16)
    o, st = _both(x, cfg)
    ref, den = oracle.batched(oracle.truncated_attention, x.q64, x.k64, x.v64, 2)
    err, _ = row_rel_err(o.cpu().numpy(), ref, den)
    assert err <= TOL_BF16, err


def test_static_workspace_rejects_a_size_beyond_the_array():
    import torch

    cfg = rs.config(5, 16, 64, 0, 1.0, rs.TAYLOR_F32)
    q = torch.zeros((1, 16, 16384, 16), device=DEV)
    v = torch.zeros((1, 16, 16384, 64), device=DEV)
    o = torch.empty_like(v)
    with pytest.raises(rs.TaylorError):
        rs.taylor_attn_prefill_into_static(q, q, v, o, None, None, cfg)
