"""GPU parity of the expanded-softmax readout (TAYLOR_READOUT_CENTERED) against the oracle.

Source: Su Jianlin, kexue.fm translation 11814, "Calculating the Gradient" and
"Linear Attention".  Prefill (float32 inputs on the feature-block kernel,
bfloat16 inputs on the pipelined kernel), decode, resume from a state written
by the truncated-kernel readout (the states are the same sums), ragged batches
and raw (un-normalised) scores.  Bars: 1e-5 relative per output row for float32
inputs; bfloat16 inputs 3e-3, as for the truncated kernel (the oracle sees the
same rounded inputs; the kernel rounds gamma_m * phi_m(sigma q) to bfloat16).  With raw
scores a row may be a small difference of larger terms (the weights go negative): there
the float32 bar is max(1e-5 ||ref_i||, 2^-18 ||M_i||), M_i the sums of absolute values of
the row's terms (oracle.centered_magnitudes).
"""

import numpy as np
import pytest

import oracle
from oracle.centered import centered_magnitudes
import recurrent_state_amd as rs
import synth
from gpu_util import TOL_F32, announce, row_rel_err, rows_within, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda"
DK, DV = 16, 64


def _cfg(order, dtype, scale=1.0):
    return rs.config(order + 1, DK, DV, 64, scale, rs.TAYLOR_BF16 if dtype == "bf16" else rs.TAYLOR_F32,
                     rs.TAYLOR_READOUT_CENTERED)


def _ref(q64, k64, v64, order, scale):
    B, H = q64.shape[:2]
    out = np.empty(q64.shape[:3] + (v64.shape[-1],))
    for b in range(B):
        for h in range(H):
            out[b, h] = oracle.centered_attention(q64[b, h], k64[b, h], v64[b, h], order, scale)
    return out


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_centered_prefill(order, dtype):
    import torch

    B, H, N = 2, 2, 700
    x = synth.make_qkv(90 + order, B, H, N, DK, DV, dtype)
    cfg = _cfg(order, dtype)
    announce("centered-prefill", order, dtype, B, H, N)
    q, k, v = x.torch(DEV)
    o = torch.empty((B, H, N, DV), device=DEV)
    st = rs.new_state(B, H, cfg, DEV)
    rs.taylor_attn_prefill(q, k, v, o, st, rs.new_workspace(cfg, B, H, N, DEV), cfg)
    err, rows = row_rel_err(o.cpu().numpy(), _ref(x.q64, x.k64, x.v64, order, 1.0))
    assert rows == B * H * N
    assert err <= tol_for(dtype), f"rel err {err:.3e}"
    # the final state is the truncated-kernel state of n = order + 1 terms
    S, z = rs.state_views(st, cfg)
    full = oracle.state(x.k64[1, 1], x.v64[1, 1], order + 1)
    got = np.concatenate([S[1, 1].cpu().numpy(), z[1, 1].cpu().numpy()[:, None]], axis=1)
    if dtype == "bf16":
        bound = 2.0**-8 * oracle.state(np.abs(x.k64[1, 1]), np.abs(x.v64[1, 1]), order + 1)
        assert np.all(np.abs(got - full) <= bound + 1e-6 * np.max(np.abs(full)))
    else:
        assert np.max(np.abs(got - full)) <= 1e-5 * np.max(np.abs(full))


@pytest.mark.parametrize("N", [1, 2, 63, 65, 129])
def test_centered_short_and_ragged_lengths(N):
    import torch

    x = synth.make_qkv(95, 1, 3, N, DK, DV)
    cfg = _cfg(2, "f32")
    announce("centered-lengths", N)
    q, k, v = x.torch(DEV)
    o = torch.empty((1, 3, N, DV), device=DEV)
    rs.taylor_attn_prefill(q, k, v, o, None, rs.new_workspace(cfg, 1, 3, N, DEV), cfg)
    err, _ = row_rel_err(o.cpu().numpy(), _ref(x.q64, x.k64, x.v64, 2, 1.0))
    assert err <= 1e-5, err


@pytest.mark.parametrize("order", [1, 2])
def test_centered_raw_scores(order):
    # un-normalised q, k with scale 1/4: the weights leave [0, 1] and some go negative
    import torch

    x = synth.make_qkv(96, 1, 2, 400, DK, DV, unit_norm=False)
    cfg = _cfg(order, "f32", 0.25)
    announce("centered-raw", order)
    q, k, v = x.torch(DEV)
    o = torch.empty((1, 2, 400, DV), device=DEV)
    rs.taylor_attn_prefill(q, k, v, o, None, rs.new_workspace(cfg, 1, 2, 400, DEV), cfg)
    ref = _ref(x.q64, x.k64, x.v64, order, 0.25)
    # per row: 1e-5 relative, or float32 rounding of the row's term magnitudes where its output is a
    # small difference of larger terms (negative weights)
    got = o.cpu().numpy()
    for h in range(2):
        mag = centered_magnitudes(x.q64[0, h], x.k64[0, h], x.v64[0, h], order, 0.25)
        r = rows_within(got[0, h], ref[0, h], mag, TOL_F32)
        assert r <= 1.0, f"head {h}: {r:.2f} x the per-row bar"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_centered_resume_from_a_kernel_readout_state(dtype):
    # A state written by the truncated-kernel readout continues under the expanded-softmax readout:
    # both read the same sums (states add across chunks, "Expanding Attention", Abstract).
    import torch

    N1, N2, H, order = 500, 333, 2, 2
    x = synth.make_qkv(97, 1, H, N1 + N2, DK, DV, dtype)
    cfg = _cfg(order, dtype)
    kcfg = rs.config(order + 1, DK, DV, 64, 1.0, cfg.in_dtype)
    announce("centered-resume", dtype)
    q, k, v = x.torch(DEV)
    st = rs.new_state(1, H, cfg, DEV)
    parts = [t[:, :, :N1].contiguous() for t in (q, k, v)]
    rs.taylor_attn_prefill(*parts, None, st, rs.new_workspace(kcfg, 1, H, N1, DEV), kcfg)
    parts = [t[:, :, N1:].contiguous() for t in (q, k, v)]
    o = torch.empty((1, H, N2, DV), device=DEV)
    rs.taylor_attn_prefill(*parts, o, st, rs.new_workspace(cfg, 1, H, N2, DEV), cfg)
    ref = _ref(x.q64, x.k64, x.v64, order, 1.0)[:, :, N1:]
    err, _ = row_rel_err(o.cpu().numpy(), ref)
    assert err <= tol_for(dtype), err


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_centered_decode(order, dtype):
    # prefill 300 tokens (state only), then 20 decode steps with the expanded-softmax readout
    import torch

    B, H, N0, T = 2, 3, 300, 20
    x = synth.make_qkv(98 + order, B, H, N0 + T, DK, DV, dtype)
    cfg = _cfg(order, dtype)
    announce("centered-decode", order, dtype)
    q, k, v = x.torch(DEV)
    st = rs.new_state(B, H, cfg, DEV)
    parts = [t[:, :, :N0].contiguous() for t in (q, k, v)]
    rs.taylor_attn_prefill(*parts, None, st, rs.new_workspace(cfg, B, H, N0, DEV), cfg)
    outs = []
    for t in range(N0, N0 + T):
        o = torch.empty((B, H, DV), device=DEV)
        rs.taylor_attn_decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(), o, st,
                                   cfg)
        outs.append(o)
    got = torch.stack(outs, dim=2).cpu().numpy()
    ref = np.empty_like(got, dtype=np.float64)
    rows = np.arange(N0, N0 + T)
    for b in range(B):
        for h in range(H):
            ref[b, h] = oracle.centered_attention_rows(x.q64[b, h], x.k64[b, h], x.v64[b, h], order, rows)
    err, _ = row_rel_err(got, ref)
    assert err <= tol_for(dtype), err


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_centered_varlen(dtype):
    import torch

    lens = [1, 63, 64, 65, 500, 0, 700]
    H, order = 2, 2
    x = synth.make_ragged(99, lens, H, DK, DV, dtype)
    cfg = _cfg(order, dtype)
    announce("centered-varlen", dtype, lens)
    q, k, v = x.torch(DEV)
    cu = x.torch_cu(DEV)
    T = sum(lens)
    o = torch.empty((H, T, DV), device=DEV)
    ws = rs.new_varlen_workspace(cfg, len(lens), H, max(lens), T, DEV)
    rs.taylor_attn_prefill_varlen(q, k, v, o, None, ws, cu, max(lens), cfg)
    got = o.cpu().numpy()
    for b, n in enumerate(lens):
        if n == 0:
            continue
        qs, ks, vs = x.seq(b)
        a = int(x.cu[b])
        for h in range(H):
            ref = oracle.centered_attention(qs[h], ks[h], vs[h], order)
            err, _ = row_rel_err(got[h, a : a + n], ref)
            assert err <= tol_for(dtype), f"sequence {b} head {h}: {err:.3e}"


def test_centered_full_size_sampled():
    # the bfloat16 prefill shape B4 x H16 x N8192, order 2: sampled rows of every head
    import torch

    B, H, N = 4, 16, 8192
    x = synth.make_qkv(3, B, H, N, DK, DV, "bf16")
    cfg = _cfg(2, "bf16")
    announce("centered-full", B, H, N)
    q, k, v = x.torch(DEV)
    o = torch.empty((B, H, N, DV), device=DEV)
    rs.taylor_attn_prefill(q, k, v, o, None, rs.new_workspace(cfg, B, H, N, DEV), cfg)
    got = o.cpu().numpy()
    rng = np.random.default_rng(300)
    for b in range(B):
        for h in range(H):
            rows = np.unique(np.concatenate([[0, 1, N - 1], rng.integers(0, N, 3)]))
            ref = oracle.centered_attention_rows(x.q64[b, h], x.k64[b, h], x.v64[b, h], 2, rows)
            err, _ = row_rel_err(got[b, h, rows], ref)
            assert err <= tol_for("bf16"), f"({b}, {h}): {err:.3e}"
