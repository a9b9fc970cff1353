"""GPU parity of taylor_attn_decode_step and taylor_state_init against the float64 oracle.

A decode step applied token by token from an empty state reproduces the causal
attention of the whole sequence (Abstract of "Expanding Attention": the
recursion is lossless with respect to the truncated kernel), and a decode that
continues a prefill state continues the same sequence.
"""

import numpy as np
import pytest

import oracle
import recurrent_state_amd as rs
import synth
from gpu_util import announce, row_rel_err, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _tokens_major(t):
    return t.permute(2, 0, 1, 3).contiguous()  # [N, B, H, d]


def _decode_all(x, cfg, state, start=0):
    import torch

    q, k, v = (_tokens_major(t) for t in x.torch(DEV))
    N, B, H = k.shape[:3]
    o = torch.empty((N, B, H, cfg.d_v), device=DEV)
    for t in range(start, N):
        rs.taylor_attn_decode_step(q[t], k[t], v[t], o[t], state, cfg)
    return o.permute(1, 2, 0, 3)[:, :, start:].cpu().numpy()


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_from_empty_state_is_causal_attention(n, dtype):
    x = synth.make_qkv(70 + n, 2, 2, 150, 16, 64, dtype)
    cfg = rs.config(n, 16, 64, 0, 1.0, rs.TAYLOR_BF16 if dtype == "bf16" else rs.TAYLOR_F32)
    announce("decode-from-zero", n, dtype)
    st = rs.new_state(2, 2, cfg, DEV)
    o = _decode_all(x, cfg, st)
    ref, den = oracle.batched(oracle.truncated_attention, x.q64, x.k64, x.v64, n)
    err, _ = row_rel_err(o, ref, den)
    assert err <= tol_for(dtype), err
    # the state after N steps is the state of the N tokens
    S, z = rs.state_views(st, cfg)
    full = oracle.state(x.k64[1, 1], x.v64[1, 1], n)
    got = np.concatenate([S[1, 1].cpu().numpy(), z[1, 1].cpu().numpy()[:, None]], axis=1)
    assert np.max(np.abs(got - full)) <= 1e-5 * np.max(np.abs(full))


@pytest.mark.parametrize("shape", [(4, 4), (8, 32), (16, 128)])
def test_decode_other_head_dims(shape):
    dk, dv = shape
    x = synth.make_qkv(80, 1, 3, 90, dk, dv)
    cfg = rs.config(3, dk, dv)
    announce("decode-dims", shape)
    st = rs.new_state(1, 3, cfg, DEV)
    o = _decode_all(x, cfg, st)
    ref, den = oracle.batched(oracle.truncated_attention, x.q64, x.k64, x.v64, 3)
    assert row_rel_err(o, ref, den)[0] <= 1e-5


@pytest.mark.parametrize("n", [2, 3, 5])
def test_decode_continues_prefill(n):
    N1, N = 1000, 1100
    x = synth.make_qkv(90 + n, 1, 4, N, 16, 64)
    cfg = rs.config(n, 16, 64, 64)
    announce("prefill+decode", n)
    q, k, v = x.torch(DEV)
    st = rs.new_state(1, 4, cfg, DEV)
    parts = [t[:, :, :N1].contiguous() for t in (k, v)]
    rs.taylor_attn_prefill(None, *parts, None, st, rs.new_workspace(cfg, 1, 4, N1, DEV), cfg)
    o = _decode_all(x, cfg, st, start=N1)
    ref, den = oracle.batched(oracle.truncated_attention, x.q64, x.k64, x.v64, n)
    err, _ = row_rel_err(o, ref[:, :, N1:], den[:, :, N1:])
    assert err <= 1e-5, err


def test_raw_scores_decode():
    x = synth.make_qkv(95, 1, 2, 120, 16, 64, unit_norm=False)
    cfg = rs.config(3, 16, 64, 0, 0.25)
    announce("decode-raw")
    st = rs.new_state(1, 2, cfg, DEV)
    o = _decode_all(x, cfg, st)
    ref, den = oracle.batched(oracle.truncated_attention, x.q64, x.k64, x.v64, 3, 0.25)
    assert row_rel_err(o, ref, den)[0] <= 1e-5


def test_state_init_zeroes_everything():
    import torch

    cfg = rs.config(3, 16, 64)
    st = torch.full((3, 5, rs.taylor_state_stride(cfg)), float("nan"), device=DEV)
    announce("state-init")
    rs.taylor_state_init(st, cfg)
    torch.cuda.synchronize()
    assert bool((st == 0).all())
