"""GPU tests of taylor_attn_prefill_into: the incoming and the final state in separate arrays.

"Expanding Attention" (Huang, arXiv:2610.20637), Abstract: the state after a call is the state
before it plus the call's own sum, so where the two live is free.  A fresh call (no incoming array)
must give exactly what zeroing a state and prefilling in place gives, and a continuation from one
array into another exactly what the in-place continuation gives, leaving the incoming array as it
was.  The arithmetic is the same in both forms, so the comparisons are bit for bit; every prefill
path is exercised (bf16 matrix-core kernel, float32 feature-block kernel with one and with several
segments per head, n = 4, the portable kernel, the expanded-softmax readout).
"""

import numpy as np
import pytest

import oracle
import recurrent_state_amd as rs
import synth
from gpu_util import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [  # (label, n, d_k, d_v, chunk, dtype, readout, B, H, N)
    ("bf16-n3", 3, 16, 64, 64, "bf16", 0, 2, 3, 700),
    ("f32-n3-segments", 3, 16, 64, 64, "f32", 0, 1, 2, 900),
    ("f32-n3-one-segment", 3, 16, 64, 64, "f32", 0, 4, 64, 128),
    ("f32-n4", 4, 16, 64, 64, "f32", 0, 1, 16, 200),
    ("portable-d8", 3, 8, 32, 64, "f32", 0, 2, 2, 300),
    ("centered-bf16", 3, 16, 64, 64, "bf16", 1, 1, 2, 500),
    ("centered-f32", 3, 16, 64, 64, "f32", 1, 1, 2, 500),
]


def _cfg(n, dk, dv, C, dtype, readout):
    return rs.config(n, dk, dv, C, 1.0, rs.TAYLOR_BF16 if dtype == "bf16" else rs.TAYLOR_F32, readout)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fresh_equals_init_then_prefill(case):
    import torch

    label, n, dk, dv, C, dtype, readout, B, H, N = case
    cfg = _cfg(n, dk, dv, C, dtype, readout)
    x = synth.make_qkv(500 + n, B, H, N, dk, dv, dtype)
    announce("prefill-into fresh", label)
    q, k, v = x.torch(DEV)
    ws = rs.new_workspace(cfg, B, H, N, DEV)
    o1 = torch.empty((B, H, N, dv), device=DEV)
    st1 = rs.new_state(B, H, cfg, DEV)
    rs.taylor_state_init(st1, cfg)
    rs.taylor_attn_prefill(q, k, v, o1, st1, ws, cfg)
    o2 = torch.empty_like(o1)
    st2 = torch.full_like(st1, float("nan"))  # never read
    rs.taylor_attn_prefill_into(q, k, v, o2, None, st2, ws, cfg)
    assert torch.equal(o1, o2)
    assert torch.equal(st1, st2)
    # state only
    st3 = torch.full_like(st1, float("nan"))
    rs.taylor_attn_prefill_into(q, k, v, None, None, st3, ws, cfg)
    S, z = rs.state_views(st3, cfg)
    ref = oracle.state(x.k64[0, 0], x.v64[0, 0], n)
    got = np.concatenate([S[0, 0].cpu().numpy(), z[0, 0].cpu().numpy()[:, None]], axis=1)
    tol = 2.0**-7 if dtype == "bf16" else 1e-5
    assert np.max(np.abs(got - ref)) <= tol * np.max(np.abs(ref))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_out_of_place_continuation(case):
    import torch

    label, n, dk, dv, C, dtype, readout, B, H, N = case
    cfg = _cfg(n, dk, dv, C, dtype, readout)
    N1 = N // 3
    x = synth.make_qkv(600 + n, B, H, N, dk, dv, dtype)
    announce("prefill-into continuation", label)
    q, k, v = x.torch(DEV)
    part = lambda t, a, b: t[:, :, a:b].contiguous()
    ws = rs.new_workspace(cfg, B, H, N, DEV)
    prefix = torch.empty(rs.new_state(B, H, cfg, DEV).shape, device=DEV)
    rs.taylor_attn_prefill_into(part(q, 0, N1), part(k, 0, N1), part(v, 0, N1), None, None, prefix, ws, cfg)
    keep = prefix.clone()
    # in place on a copy, and out of place from the cached prefix
    inplace = prefix.clone()
    o1 = torch.empty((B, H, N - N1, dv), device=DEV)
    rs.taylor_attn_prefill(part(q, N1, N), part(k, N1, N), part(v, N1, N), o1, inplace, ws, cfg)
    out = torch.full_like(prefix, float("nan"))
    o2 = torch.empty_like(o1)
    rs.taylor_attn_prefill_into(part(q, N1, N), part(k, N1, N), part(v, N1, N), o2, prefix, out, ws, cfg)
    assert torch.equal(prefix, keep), "the incoming state changed"
    assert torch.equal(o1, o2)
    assert torch.equal(inplace, out)


def test_no_tokens_copies_or_zeroes():
    import torch

    cfg = _cfg(3, 16, 64, 64, "bf16", 0)
    announce("prefill-into N=0")
    x = synth.make_qkv(700, 2, 3, 100, 16, 64, "bf16")
    q, k, v = x.torch(DEV)
    src = torch.empty(rs.new_state(2, 3, cfg, DEV).shape, device=DEV)
    rs.taylor_attn_prefill_into(q, k, v, None, None, src, rs.new_workspace(cfg, 2, 3, 100, DEV), cfg)
    empty = [t[:, :, :0].contiguous() for t in (q, k, v)]
    dst = torch.full_like(src, float("nan"))
    rs.taylor_attn_prefill_into(*empty, None, src, dst, None, cfg)
    assert torch.equal(dst, src)
    rs.taylor_attn_prefill_into(*empty, None, None, dst, None, cfg)
    assert bool((dst == 0).all())


RAGGED = [  # (label, n, dtype, lengths)
    ("bf16-n3", 3, "bf16", [1, 63, 0, 700, 65, 5]),
    ("f32-n3", 3, "f32", [200, 0, 31, 333]),
    ("f32-n5", 5, "f32", [70, 0, 130]),
    ("tiny", 3, "f32", [5, 0, 9]),  # a batch shorter than one chunk
]


@pytest.mark.parametrize("case", RAGGED, ids=[c[0] for c in RAGGED])
def test_varlen_into(case):
    # fresh = init + prefill, and out of place = in place, bit for bit, empty sequences included
    import torch

    label, n, dtype, lens = case
    H = 2
    cfg = _cfg(n, 16, 64, 64, dtype, 0)
    x = synth.make_ragged(800 + n, lens, H, 16, 64, dtype)
    announce("varlen-into", label, lens)
    q, k, v = x.torch(DEV)
    cu = x.torch_cu(DEV)
    T, N = sum(lens), max(lens)
    ws = rs.new_varlen_workspace(cfg, len(lens), H, N, T, DEV)
    shape = (len(lens), H, rs.taylor_state_stride(cfg))
    o1 = torch.empty((H, T, 64), device=DEV)
    st1 = torch.empty(shape, device=DEV)
    rs.taylor_state_init(st1, cfg)
    rs.taylor_attn_prefill_varlen(q, k, v, o1, st1, ws, cu, N, cfg)
    o2 = torch.empty_like(o1)
    st2 = torch.full(shape, float("nan"), device=DEV)
    rs.taylor_attn_prefill_varlen_into(q, k, v, o2, None, st2, ws, cu, N, cfg)
    assert torch.equal(o1, o2)
    assert torch.equal(st1, st2)
    # continue the same batch from those states: in place on a copy, and out of place
    inplace = st1.clone()
    rs.taylor_attn_prefill_varlen(q, k, v, o1, inplace, ws, cu, N, cfg)
    keep = st1.clone()
    out = torch.full(shape, float("nan"), device=DEV)
    rs.taylor_attn_prefill_varlen_into(q, k, v, o2, st1, out, ws, cu, N, cfg)
    assert torch.equal(st1, keep), "the incoming states changed"
    assert torch.equal(o1, o2)
    assert torch.equal(inplace, out)


@pytest.mark.parametrize("n,B,H,N", [(3, 2, 128, 1000), (3, 4, 16, 300), (2, 4, 16, 300), (1, 4, 16, 300)])
def test_one_pass_bf16(n, B, H, N):
    # Shapes the bfloat16 kernel runs in one pass per (sequence, head) pair (no state pass, no scan):
    # 256 pairs at 16 chunks, and 64 short pairs at n = 1, 2, 3.  Outputs and final states against the oracle on
    # sampled heads; state-only = the full call's state, in place = out of place, bit for bit; the
    # padding after z is written as zeros.
    import torch

    cfg = _cfg(n, 16, 64, 128, "bf16", 0)
    x = synth.make_qkv(910 + n, B, H, N, 16, 64, "bf16")
    announce("prefill one pass", n, B, H, N)
    q, k, v = x.torch(DEV)
    ws = rs.new_workspace(cfg, B, H, N, DEV)
    o = torch.empty((B, H, N, 64), device=DEV)
    st = torch.full(rs.new_state(B, H, cfg, DEV).shape, float("nan"), device=DEV)
    rs.taylor_attn_prefill_into(q, k, v, o, None, st, ws, cfg)
    W = rs.taylor_feature_width(n, 16)
    assert bool((st[:, :, W * 65:] == 0).all())
    S, z = rs.state_views(st, cfg)
    for b, h in [(0, 0), (B - 1, H // 2 + 1), (B - 1, H - 1)]:
        ref, den = oracle.truncated_attention(x.q64[b, h], x.k64[b, h], x.v64[b, h], n)
        err = np.max(np.abs(o[b, h].cpu().numpy() - ref) / np.max(np.abs(ref), axis=1, keepdims=True))
        assert err <= 3e-3, f"head ({b}, {h}): rel err {err:.3e}"
        sref = oracle.state(x.k64[b, h], x.v64[b, h], n)
        got = np.concatenate([S[b, h].cpu().numpy(), z[b, h].cpu().numpy()[:, None]], axis=1)
        assert np.max(np.abs(got - sref)) <= 2.0**-7 * np.max(np.abs(sref))
    st_only = torch.full_like(st, float("nan"))
    rs.taylor_attn_prefill_into(q, k, v, None, None, st_only, ws, cfg)
    assert torch.equal(st_only, st)
    # continuation: in place and out of place from a cached prefix
    N1 = N // 3
    part = lambda t, a, e: t[:, :, a:e].contiguous()
    prefix = torch.empty_like(st)
    rs.taylor_attn_prefill_into(part(q, 0, N1), part(k, 0, N1), part(v, 0, N1), None, None, prefix, ws, cfg)
    keep = prefix.clone()
    inplace = prefix.clone()
    o1 = torch.empty((B, H, N - N1, 64), device=DEV)
    rs.taylor_attn_prefill(part(q, N1, N), part(k, N1, N), part(v, N1, N), o1, inplace, ws, cfg)
    out = torch.full_like(prefix, float("nan"))
    o2 = torch.empty_like(o1)
    rs.taylor_attn_prefill_into(part(q, N1, N), part(k, N1, N), part(v, N1, N), o2, prefix, out, ws, cfg)
    assert torch.equal(prefix, keep), "the incoming state changed"
    assert torch.equal(o1, o2)
    assert torch.equal(inplace, out)
    b, h = B - 1, H - 1
    ref, _ = oracle.truncated_attention(x.q64[b, h], x.k64[b, h], x.v64[b, h], n)
    err = np.max(np.abs(o2[b, h].cpu().numpy() - ref[N1:]) / np.max(np.abs(ref[N1:]), axis=1, keepdims=True))
    assert err <= 3e-3, f"continuation: rel err {err:.3e}"


@pytest.mark.parametrize("seed,n_seqs,hi", [(921, 40, 300), (922, 100, 120)])
def test_one_pass_ragged_bf16(seed, n_seqs, hi):
    # Ragged batches the bfloat16 kernel runs in one pass per (sequence, head) pair (short sequences,
    # some empty, 8 heads; 40 of up to 300 tokens are taken longest first, 100 of up to 120 in order):
    # outputs and final states against the oracle on sampled pairs; fresh = init + prefill and out of
    # place = in place, bit for bit; an empty sequence's final state is its incoming one (zero when
    # fresh), padding zeroed.
    import torch

    H = 8
    lens = synth.ragged_lengths(seed, n_seqs, 1, hi)
    lens[3] = lens[17] = 0
    lens[-1] = 0
    cfg = _cfg(3, 16, 64, 64, "bf16", 0)
    x = synth.make_ragged(seed, lens, H, 16, 64, "bf16")
    announce("varlen one pass", len(lens), H, max(lens))
    q, k, v = x.torch(DEV)
    cu = x.torch_cu(DEV)
    T, N = sum(lens), max(lens)
    ws = rs.new_varlen_workspace(cfg, len(lens), H, N, T, DEV)
    shape = (len(lens), H, rs.taylor_state_stride(cfg))
    o = torch.empty((H, T, 64), device=DEV)
    st = torch.full(shape, float("nan"), device=DEV)
    rs.taylor_attn_prefill_varlen_into(q, k, v, o, None, st, ws, cu, N, cfg)
    W = rs.taylor_feature_width(3, 16)
    assert bool((st[:, :, W * 65:] == 0).all())
    assert bool((st[3] == 0).all()) and bool((st[-1] == 0).all())
    S, z = rs.state_views(st, cfg)
    cuh = np.concatenate([[0], np.cumsum(lens)])
    b_long = int(np.argmax(lens))
    for b, h in [(0, 0), (b_long, H - 1), (len(lens) - 2, 3)]:
        a, e = cuh[b], cuh[b + 1]
        ref, _ = oracle.truncated_attention(x.q64[h, a:e], x.k64[h, a:e], x.v64[h, a:e], 3)
        err = np.max(np.abs(o[h, a:e].cpu().numpy() - ref) / np.max(np.abs(ref), axis=1, keepdims=True))
        assert err <= 3e-3, f"pair ({b}, {h}): rel err {err:.3e}"
        sref = oracle.state(x.k64[h, a:e], x.v64[h, a:e], 3)
        got = np.concatenate([S[b, h].cpu().numpy(), z[b, h].cpu().numpy()[:, None]], axis=1)
        assert np.max(np.abs(got - sref)) <= 2.0**-7 * np.max(np.abs(sref))
    st1 = torch.empty(shape, device=DEV)
    rs.taylor_state_init(st1, cfg)
    o1 = torch.empty_like(o)
    rs.taylor_attn_prefill_varlen(q, k, v, o1, st1, ws, cu, N, cfg)
    assert torch.equal(o1, o)
    assert torch.equal(st1, st)
    inplace = st1.clone()
    rs.taylor_attn_prefill_varlen(q, k, v, o1, inplace, ws, cu, N, cfg)
    keep = st1.clone()
    out = torch.full(shape, float("nan"), device=DEV)
    o2 = torch.empty_like(o)
    rs.taylor_attn_prefill_varlen_into(q, k, v, o2, st1, out, ws, cu, N, cfg)
    assert torch.equal(st1, keep), "the incoming states changed"
    assert torch.equal(o1, o2)
    assert torch.equal(inplace, out)
    assert torch.equal(out[3], st1[3]) and torch.equal(out[17], st1[17])


def test_split_rounds_bf16():
    # 96 pairs x 4,096 tokens: split into two segments per pair (192 workgroups, one round; the ceiling
    # of 256 / 96 = 3 would spill a second round), state pass + scan + readout.  Sampled heads against
    # the oracle, outputs and final states.
    import torch

    B, H, N = 6, 16, 4096
    cfg = _cfg(3, 16, 64, 128, "bf16", 0)
    x = synth.make_qkv(930, B, H, N, 16, 64, "bf16")
    announce("prefill split rounds", B, H, N)
    q, k, v = x.torch(DEV)
    ws = rs.new_workspace(cfg, B, H, N, DEV)
    o = torch.empty((B, H, N, 64), device=DEV)
    st = torch.full(rs.new_state(B, H, cfg, DEV).shape, float("nan"), device=DEV)
    rs.taylor_attn_prefill_into(q, k, v, o, None, st, ws, cfg)
    S, z = rs.state_views(st, cfg)
    for b, h in [(0, 1), (B - 1, H - 2)]:
        ref, _ = oracle.truncated_attention(x.q64[b, h], x.k64[b, h], x.v64[b, h], 3)
        err = np.max(np.abs(o[b, h].cpu().numpy() - ref) / np.max(np.abs(ref), axis=1, keepdims=True))
        assert err <= 3e-3, f"head ({b}, {h}): rel err {err:.3e}"
        sref = oracle.state(x.k64[b, h], x.v64[b, h], 3)
        got = np.concatenate([S[b, h].cpu().numpy(), z[b, h].cpu().numpy()[:, None]], axis=1)
        assert np.max(np.abs(got - sref)) <= 2.0**-7 * np.max(np.abs(sref))
