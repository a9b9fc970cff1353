"""GPU parity of taylor_attn_prefill_backward against the float64 oracle's gradients (n = 1..3 on the
segment kernels, n = 4, 5 on the feature-block kernels).

The oracle's gradients are pinned by finite differences of the forward definition
(tests/test_oracle_backward.py).  The kernels compute in float32 from the same
(rounded) inputs, so both input types share the bar, compared row by row (one
token's dq, dk or dv): ||got_i - ref_i|| <= max(1e-5 ||ref_i||, 2^-18 ||M_i||), where
M_i holds the sums of absolute values of the row's terms (the oracle's magnitudes).
The second term is the float32 rounding of a row that is a small difference of
large terms (dq of the first tokens, raw scores, a scale that is not a power of two);
it is 64 unit roundoffs of the terms, not a looser relative bar.  The forward
outputs o given to the backward are the oracle's, rounded to float32, so that the
check isolates the backward; one case feeds the library's own forward outputs.
"""

import numpy as np
import pytest

import oracle
import recurrent_state_amd as rs
import synth
from gpu_util import TOL_F32, announce, rows_within

pytestmark = pytest.mark.gpu
DEV = "cuda"
DK, DV = 16, 64


def _rel(got, ref):
    # relative Frobenius error (the incoming state's gradient, a [W, d_v + 1] block per head)
    return float(np.linalg.norm(np.asarray(got, dtype=np.float64) - ref) / np.linalg.norm(ref))


def _cfg(n, dtype, scale=1.0):
    return rs.config(n, DK, DV, 64, scale, rs.TAYLOR_BF16 if dtype == "bf16" else rs.TAYLOR_F32)


def _grad_inputs(x, seed):
    B, H, N = x.k64.shape[:3]
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, H, N, DV)).astype(np.float32)


def _run(x, g, o, cfg, state=None, dstate=None):
    import torch

    q, k, v = x.torch(DEV)
    B, H, N = k.shape[:3]
    dq = torch.empty((B, H, N, DK), device=DEV)
    dk = torch.empty((B, H, N, DK), device=DEV)
    dv = torch.empty((B, H, N, DV), device=DEV)
    ws = rs.new_backward_workspace(cfg, B, H, N, DEV)
    rs.taylor_attn_prefill_backward(q, k, v, torch.from_numpy(o).to(DEV), torch.from_numpy(g).to(DEV), state, dstate,
                                    dq, dk, dv, ws, cfg)
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def _oracle_fwd(x, n, scale):
    o, _ = oracle.batched(oracle.truncated_attention, x.q64, x.k64, x.v64, n, scale)
    return o


def _check(got, x, g, n, scale, tol=TOL_F32, label=""):
    B, H = x.k64.shape[:2]
    for b in range(B):
        for h in range(H):
            args = (x.q64[b, h], x.k64[b, h], x.v64[b, h], g[b, h].astype(np.float64), n, scale)
            ref = oracle.attention_backward(*args)
            mag = oracle.attention_backward_magnitudes(*args)
            for name, gt, rf, mg in zip(("dq", "dk", "dv"), got, ref, mag):
                if n == 1 and name != "dv":
                    assert np.all(gt[b, h] == 0), f"{label} {name} ({b}, {h}) nonzero at n = 1"
                    continue
                r = rows_within(gt[b, h], rf, mg, tol)
                assert r <= 1.0, f"{label} {name} ({b}, {h}): {r:.2f} x the per-row bar"


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_matches_oracle(n, dtype):
    x = synth.make_qkv(110 + n, 2, 2, 333, DK, DV, dtype)
    g = _grad_inputs(x, 1100 + n)
    cfg = _cfg(n, dtype)
    announce("backward", n, dtype, 333)
    o = _oracle_fwd(x, n, 1.0).astype(np.float32)
    _check(_run(x, g, o, cfg), x, g, n, 1.0, label="backward")


@pytest.mark.parametrize("N", [1, 15, 16, 17, 100])
def test_backward_short_lengths(N):
    x = synth.make_qkv(115, 1, 3, N, DK, DV)
    g = _grad_inputs(x, 1150 + N)
    cfg = _cfg(3, "f32")
    announce("backward-lengths", N)
    o = _oracle_fwd(x, 3, 1.0).astype(np.float32)
    _check(_run(x, g, o, cfg), x, g, 3, 1.0, label=f"N={N}")


@pytest.mark.parametrize("n", [4, 5])
@pytest.mark.parametrize("N", [1, 31, 32, 33, 64, 97])
def test_backward_feature_blocks_short_lengths(n, N):
    # n = 4, 5 walk 32-token chunks over feature blocks: lengths at and around chunk edges
    x = synth.make_qkv(130 + n, 1, 3, N, DK, DV)
    g = _grad_inputs(x, 1300 + N)
    cfg = _cfg(n, "f32")
    announce("backward-blocks-lengths", n, N)
    o = _oracle_fwd(x, n, 1.0).astype(np.float32)
    _check(_run(x, g, o, cfg), x, g, n, 1.0, label=f"n={n} N={N}")


@pytest.mark.parametrize("n", [4, 5])
def test_backward_feature_blocks_raw_scores_and_many_heads(n):
    # raw Gaussian q, k at sigma = 1/4 (large, cancelling terms), bf16 inputs, 2 x 5 heads
    x = synth.make_qkv(135 + n, 2, 5, 200, DK, DV, "bf16", unit_norm=False)
    g = _grad_inputs(x, 1350 + n)
    cfg = _cfg(n, "bf16", 0.25)
    announce("backward-blocks-raw", n)
    o = _oracle_fwd(x, n, 0.25).astype(np.float32)
    _check(_run(x, g, o, cfg), x, g, n, 0.25, label=f"raw n={n}")


@pytest.mark.parametrize("n", [4, 5])
def test_backward_feature_blocks_bitwise_repeatable(n):
    # per-block gradient parts summed in block order (the last block adds the intra-chunk parts): two
    # calls on the same inputs give the same bits
    x = synth.make_qkv(140 + n, 1, 3, 333, DK, DV)
    g = _grad_inputs(x, 1400 + n)
    cfg = _cfg(n, "f32")
    announce("backward-blocks-repeat", n)
    o = _oracle_fwd(x, n, 1.0).astype(np.float32)
    first, second = _run(x, g, o, cfg), _run(x, g, o, cfg)
    for name, a, b in zip(("dq", "dk", "dv"), first, second):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{name} not bitwise repeatable"


def test_backward_raw_scores():
    x = synth.make_qkv(116, 1, 2, 300, DK, DV, unit_norm=False)
    g = _grad_inputs(x, 1160)
    cfg = _cfg(3, "f32", 0.25)
    announce("backward-raw")
    o = _oracle_fwd(x, 3, 0.25).astype(np.float32)
    _check(_run(x, g, o, cfg), x, g, 3, 0.25, label="raw")


def test_backward_bf16_scale_not_a_power_of_two():
    # bfloat16 inputs take exact bfloat16 products for the state (k, v are exact) while a = sigma q is
    # not exact at sigma = 0.3: the float32 paths for everything a enters
    x = synth.make_qkv(121, 1, 2, 300, DK, DV, "bf16", unit_norm=False)
    g = _grad_inputs(x, 1210)
    cfg = _cfg(3, "bf16", 0.3)
    announce("backward-bf16-scale")
    o = _oracle_fwd(x, 3, 0.3).astype(np.float32)
    _check(_run(x, g, o, cfg), x, g, 3, 0.3, label="bf16 sigma 0.3")


def test_backward_with_the_library_forward():
    # end to end: the library's own float32 forward outputs feed the backward
    import torch

    n, B, H, N = 3, 1, 4, 2048
    x = synth.make_qkv(117, B, H, N, DK, DV)
    g = _grad_inputs(x, 1170)
    cfg = _cfg(n, "f32")
    announce("backward-e2e", N)
    q, k, v = x.torch(DEV)
    o = torch.empty((B, H, N, DV), device=DEV)
    rs.taylor_attn_prefill(q, k, v, o, None, rs.new_workspace(cfg, B, H, N, DEV), cfg)
    _check(_run(x, g, o.cpu().numpy(), cfg), x, g, n, 1.0, label="e2e")


@pytest.mark.parametrize("n,N", [(3, 300), (3, 50), (4, 300), (5, 77)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_from_a_state_and_its_gradient(dtype, n, N):
    # the forward continued from an incoming state: gradients of q, k, v and of that state (n = 3,
    # N = 50: one segment, where no state pass runs; n = 4, 5: the feature-block kernels)
    import torch

    H, N0 = 2, 200
    x0 = synth.make_qkv(118, 1, H, N0, DK, DV, dtype)
    x = synth.make_qkv(119, 1, H, N, DK, DV, dtype)
    g = _grad_inputs(x, 1190)
    cfg = _cfg(n, dtype)
    announce("backward-state", dtype, N)
    st0 = np.stack([oracle.state(x0.k64[0, h], x0.v64[0, h], n) for h in range(H)])  # [H, W, 65]
    stride = rs.taylor_state_stride(cfg)
    W = st0.shape[1]
    flat = np.zeros((1, H, stride), dtype=np.float32)
    flat[0, :, : W * DV] = st0[:, :, :DV].reshape(H, -1)
    flat[0, :, W * DV : W * (DV + 1)] = st0[:, :, DV]
    o = np.empty((1, H, N, DV), dtype=np.float32)
    refs = []
    for h in range(H):
        oh, _ = oracle.recurrent(x.q64[0, h], x.k64[0, h], x.v64[0, h], n, 1.0, st0[h])
        o[0, h] = oh
        refs.append(oracle.attention_backward_from_state(x.q64[0, h], x.k64[0, h], x.v64[0, h], g[0, h], n, 1.0, st0[h]))
    state = torch.from_numpy(flat).to(DEV)
    dstate = torch.zeros_like(state)
    got = _run(x, g, o, cfg, state, dstate)
    ds = dstate.cpu().numpy()
    for h in range(H):
        mags = oracle.attention_backward_magnitudes(x.q64[0, h], x.k64[0, h], x.v64[0, h], g[0, h], n, 1.0, st0[h])
        for name, gt, rf, mg in zip(("dq", "dk", "dv"), (a[0, h] for a in got), refs[h][:3], mags[:3]):
            r = rows_within(gt, rf, mg, TOL_F32)
            assert r <= 1.0, f"{name} head {h}: {r:.2f} x the per-row bar"
        want = refs[h][3]
        gs = np.concatenate([ds[0, h, : W * DV].reshape(W, DV), ds[0, h, W * DV : W * (DV + 1)][:, None]], axis=1)
        assert _rel(gs, want) <= 1e-5, f"dstate head {h}: {_rel(gs, want):.3e}"


@pytest.mark.parametrize("n", [3, 4, 5])
def test_backward_in_pieces_passes_the_state_gradient(n):
    # A sequence prefilled in two calls is differentiated in reverse: the second call's backward
    # returns dL/d(state between the calls), which seeds the first call's backward.
    import torch

    H, N1, N2 = 2, 400, 250
    x = synth.make_qkv(120, 1, H, N1 + N2, DK, DV)
    g = _grad_inputs(x, 1200)
    cfg = _cfg(n, "f32")
    announce("backward-pieces")
    o = _oracle_fwd(x, n, 1.0).astype(np.float32)
    q, k, v = x.torch(DEV)
    st = rs.new_state(1, H, cfg, DEV)
    parts1 = [t[:, :, :N1].contiguous() for t in (q, k, v)]
    o1 = torch.empty((1, H, N1, DV), device=DEV)
    rs.taylor_attn_prefill(*parts1, o1, st, rs.new_workspace(cfg, 1, H, N1, DEV), cfg)  # st = state after piece 1
    outs = []
    dstate = torch.zeros_like(st)
    for lo, hi, state in ((N1, N1 + N2, st), (0, N1, None)):
        parts = [t[:, :, lo:hi].contiguous() for t in (q, k, v)]
        dq = torch.empty((1, H, hi - lo, DK), device=DEV)
        dk = torch.empty((1, H, hi - lo, DK), device=DEV)
        dv = torch.empty((1, H, hi - lo, DV), device=DEV)
        rs.taylor_attn_prefill_backward(*parts, torch.from_numpy(o[:, :, lo:hi].copy()).to(DEV),
                                        torch.from_numpy(g[:, :, lo:hi].copy()).to(DEV), state, dstate, dq, dk, dv,
                                        rs.new_backward_workspace(cfg, 1, H, hi - lo, DEV), cfg)
        outs.append((dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()))
    got = [np.concatenate([outs[1][i], outs[0][i]], axis=2) for i in range(3)]
    _check(got, x, g, n, 1.0, label="pieces")


def test_backward_full_size_properties():
    # the bfloat16 prefill shape B4 x H16 x N8192: finite gradients, the sum rule of dv (each output is
    # an average: sum_j dv_j = sum_i g_i) and sampled rows of dq against the oracle
    import torch

    n, B, H, N = 3, 4, 16, 8192
    x = synth.make_qkv(3, B, H, N, DK, DV, "bf16")
    cfg = _cfg(n, "bf16")
    announce("backward-full", B, H, N)
    q, k, v = x.torch(DEV)
    # forward outputs from the float32 kernels on the same (exactly widened) inputs, so that the
    # sampled rows below see float32-accurate o
    f32 = _cfg(n, "f32")
    o = torch.empty((B, H, N, DV), device=DEV)
    rs.taylor_attn_prefill(q.float(), k.float(), v.float(), o, None, rs.new_workspace(f32, B, H, N, DEV), f32)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1210)
    g = torch.randn((B, H, N, DV), generator=gen, device=DEV)
    dq = torch.empty((B, H, N, DK), device=DEV)
    dk = torch.empty((B, H, N, DK), device=DEV)
    dv = torch.empty((B, H, N, DV), device=DEV)
    rs.taylor_attn_prefill_backward(q, k, v, o, g, None, None, dq, dk, dv, rs.new_backward_workspace(cfg, B, H, N, DEV),
                                    cfg)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    sdv = dv.double().sum(dim=2)
    sg = g.double().sum(dim=2)
    assert float((sdv - sg).abs().max()) <= 1e-3 * float(sg.abs().max())
    gn = g.cpu().numpy()
    dqn = dq.cpu().numpy()
    rng = np.random.default_rng(1211)
    for b, h in ((0, 0), (3, 15), (1, 7)):
        rows = np.unique(np.concatenate([[0, 1, 63, 64, N - 1], rng.integers(1, N, 4)]))
        args = (x.q64[b, h], x.k64[b, h], x.v64[b, h], gn[b, h], n, rows)
        ref = oracle.attention_backward_dq_rows(*args)
        mag = oracle.attention_backward_dq_magnitude_rows(*args)
        r = rows_within(dqn[b, h, rows], ref, mag, TOL_F32)
        assert r <= 1.0, f"dq rows ({b}, {h}): {r:.2f} x the per-row bar"


@pytest.mark.parametrize("n", [4, 5])
def test_backward_feature_blocks_full_size_properties(n):
    # the order-sweep shape B1 x H16 x N16384 (float32) on the feature-block kernels: finite gradients,
    # the sum rule of dv and sampled rows of dq against the oracle
    import torch

    B, H, N = 1, 16, 16384
    x = synth.make_qkv(5, B, H, N, DK, DV)
    cfg = _cfg(n, "f32")
    announce("backward-blocks-full", n, B, H, N)
    q, k, v = x.torch(DEV)
    o = torch.empty((B, H, N, DV), device=DEV)
    rs.taylor_attn_prefill(q, k, v, o, None, rs.new_workspace(cfg, B, H, N, DEV), cfg)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1220 + n)
    g = torch.randn((B, H, N, DV), generator=gen, device=DEV)
    dq = torch.empty((B, H, N, DK), device=DEV)
    dk = torch.empty((B, H, N, DK), device=DEV)
    dv = torch.empty((B, H, N, DV), device=DEV)
    rs.taylor_attn_prefill_backward(q, k, v, o, g, None, None, dq, dk, dv, rs.new_backward_workspace(cfg, B, H, N, DEV),
                                    cfg)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    sdv = dv.double().sum(dim=2)
    sg = g.double().sum(dim=2)
    assert float((sdv - sg).abs().max()) <= 1e-3 * float(sg.abs().max())
    gn = g.cpu().numpy()
    dqn = dq.cpu().numpy()
    rng = np.random.default_rng(1230 + n)
    for h in (0, 7, 15):
        rows = np.unique(np.concatenate([[0, 1, 31, 32, 33, N - 1], rng.integers(1, N, 4)]))
        args = (x.q64[0, h], x.k64[0, h], x.v64[0, h], gn[0, h], n, rows)
        ref = oracle.attention_backward_dq_rows(*args)
        mag = oracle.attention_backward_dq_magnitude_rows(*args)
        r = rows_within(dqn[0, h, rows], ref, mag, TOL_F32)
        assert r <= 1.0, f"dq rows head {h}: {r:.2f} x the per-row bar"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_state", [False, True])
def test_autograd_op(dtype, with_state):
    # rs.taylor_attention under torch.autograd: the gradients equal the explicit entry points' (bit for
    # bit, cast to the input type), and for float32 inputs the oracle's gradients
    import torch

    n, B, H, N = 3, 1, 2, 300
    cfg = _cfg(n, dtype)
    x = synth.make_qkv(125, B, H, N, DK, DV, dtype)
    g = _grad_inputs(x, 1250)
    announce("autograd op", dtype, with_state)
    q, k, v = (t.clone().requires_grad_(True) for t in x.torch(DEV))
    state = None
    if with_state:
        x0 = synth.make_qkv(126, B, H, 200, DK, DV, dtype)
        st0 = torch.empty(rs.new_state(B, H, cfg, DEV).shape, device=DEV)
        rs.taylor_attn_prefill_into(*x0.torch(DEV), None, None, st0, rs.new_workspace(cfg, B, H, 200, DEV), cfg)
        state = st0.clone().requires_grad_(True)
    o = rs.taylor_attention(q, k, v, cfg, state)
    gt = torch.from_numpy(g).to(DEV)
    (o * gt).sum().backward()
    # the explicit calls
    qd, kd, vd = x.torch(DEV)
    o2 = torch.empty_like(o)
    rs.taylor_attn_prefill_into(qd, kd, vd, o2, None if state is None else state.detach(), None,
                                rs.new_workspace(cfg, B, H, N, DEV), cfg)
    assert torch.equal(o.detach(), o2)
    dq = torch.empty((B, H, N, DK), device=DEV)
    dk = torch.empty_like(dq)
    dv = torch.empty((B, H, N, DV), device=DEV)
    ds = None if state is None else torch.zeros_like(state)
    rs.taylor_attn_prefill_backward(qd, kd, vd, o2, gt, None if state is None else state.detach(), ds, dq, dk, dv,
                                    rs.new_backward_workspace(cfg, B, H, N, DEV), cfg)
    assert torch.equal(q.grad, dq.to(q.dtype)) and torch.equal(k.grad, dk.to(k.dtype))
    assert torch.equal(v.grad, dv.to(v.dtype))
    if state is not None:
        assert torch.equal(state.grad, ds)
    if dtype == "f32" and state is None:
        _check([t.cpu().numpy() for t in (q.grad, k.grad, v.grad)], x, g, n, 1.0, label="autograd")
