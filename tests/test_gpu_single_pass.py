"""GPU tests of the single-pass prefill over segments (state sums, look-back and readout in one launch).

"Expanding Attention" (Huang, arXiv:2610.20637), Abstract: the states add across chunks, so prefill
admits a parallel scan; here the scan is a decoupled look-back between the segments of each
(sequence, head) pair.  Equal-length bfloat16 calls that split pairs into segments take this form.
Checked: the oracle at the segmented shapes (64 and 96 pairs of 8,192 tokens; 8 pairs of 777 tokens
cut into many one-chunk segments; 2 pairs of 16,384 and one of 65,536 tokens in 128 and 256 segments), continuation from a state in place and out of place, a workspace
reused by calls of other shapes or holding arbitrary bytes (a flag from another call must read as
unpublished), and graph replays (the recorded form clears its flags first) interleaved with eager
calls on the same workspace.
"""

import numpy as np
import pytest

import oracle
import recurrent_state_amd as rs
import synth
from gpu_util import TOL_BF16, announce, row_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cfg(n=3):
    return rs.config(n, 16, 64, 0, 1.0, rs.TAYLOR_BF16)


def _rows(N, seed):
    rng = np.random.default_rng(seed)
    edges = [0, 1, 63, 64, N // 4 - 1, N // 4, N // 2 - 1, N // 2, 3 * N // 4, N - 1]
    return sorted(set(r for r in edges if 0 <= r < N) | set(int(r) for r in rng.integers(0, N, 6)))


def _check_oracle(x, o, st, heads, n=3, full=False):
    S, z = rs.state_views(st, _cfg(n))
    for b, h in heads:
        if full:
            ref, den = oracle.truncated_attention(x.q64[b, h], x.k64[b, h], x.v64[b, h], n)
            err, _ = row_rel_err(o[b, h].cpu().numpy(), ref, den)
        else:
            rows = _rows(x.k64.shape[2], 17 * b + h)
            ref, den = oracle.truncated_attention_rows(x.q64[b, h], x.k64[b, h], x.v64[b, h], n, rows)
            err, _ = row_rel_err(o[b, h, rows].cpu().numpy(), ref, den)
        assert err <= TOL_BF16, f"({b}, {h}): {err:.3e}"
        # final state entry by entry: bfloat16 features (2^-9) summed in float32, bar 2^-8 sum |phi||v|
        want = oracle.state(x.k64[b, h], x.v64[b, h], n)
        bound = 2.0**-8 * oracle.state(np.abs(x.k64[b, h]), np.abs(x.v64[b, h]), n)
        got = np.concatenate([S[b, h].cpu().numpy(), z[b, h].cpu().numpy()[:, None]], axis=1)
        assert np.all(np.abs(got - want) <= bound), f"state ({b}, {h})"


# (2, 1, 16384) and (1, 1, 65536): 128 and 256 segments per pair, so the look-back of segments past the
# 64th reads its flags in more than one window of 64
@pytest.mark.parametrize("B,H,N", [(4, 16, 8192), (6, 16, 8192), (2, 4, 777), (2, 1, 16384), (1, 1, 65536)])
def test_segmented_shapes_against_the_oracle(B, H, N):
    import torch

    cfg = _cfg()
    x = synth.make_qkv(960, B, H, N, 16, 64, "bf16")
    announce("single-pass", B, H, N)
    q, k, v = x.torch(DEV)
    o = torch.full((B, H, N, 64), float("nan"), device=DEV)
    st = torch.full((B, H, rs.taylor_state_stride(cfg)), float("nan"), device=DEV)
    rs.taylor_attn_prefill_into(q, k, v, o, None, st, rs.new_workspace(cfg, B, H, N, DEV), cfg)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(st).all())
    _check_oracle(x, o, st, [(0, 0), (B - 1, H - 1), (B // 2, H // 2)], full=N <= 1024)


@pytest.mark.parametrize("n", [1, 2, 3])
def test_continuation_in_place_and_out_of_place(n):
    # prefill N1 tokens, then N2 more from that state: in place (state_in == state_out) and into a
    # separate array (the incoming one left as it was) give the same bits, and both match the oracle
    # over all N1 + N2 tokens
    import torch

    B, H, N1, N2 = 2, 16, 3000, 5000
    cfg = _cfg(n)
    x = synth.make_qkv(961 + n, B, H, N1 + N2, 16, 64, "bf16")
    announce("single-pass continuation", n)
    q, k, v = x.torch(DEV)
    a = [t[:, :, :N1].contiguous() for t in (q, k, v)]
    b = [t[:, :, N1:].contiguous() for t in (q, k, v)]
    stride = rs.taylor_state_stride(cfg)
    st0 = torch.empty((B, H, stride), device=DEV)
    rs.taylor_attn_prefill_into(*a, None, None, st0, rs.new_workspace(cfg, B, H, N1, DEV), cfg)
    ws = rs.new_workspace(cfg, B, H, N2, DEV)
    st_in = st0.clone()
    o1 = torch.empty((B, H, N2, 64), device=DEV)
    rs.taylor_attn_prefill_into(*b, o1, st_in, st_in, ws, cfg)
    st_out = torch.full_like(st0, float("nan"))
    o2 = torch.empty_like(o1)
    rs.taylor_attn_prefill_into(*b, o2, st0, st_out, ws, cfg)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(st_in, st_out)
    full_o = torch.cat([torch.zeros((B, H, N1, 64), device=DEV), o2], dim=2)
    S, z = rs.state_views(st_out, cfg)
    for bb, h in [(0, 3), (1, 15)]:
        rows = [N1, N1 + 1, N1 + 2047, N1 + 2048, N1 + N2 - 1] + list(range(N1 + 4000, N1 + 4004))
        ref, den = oracle.truncated_attention_rows(x.q64[bb, h], x.k64[bb, h], x.v64[bb, h], n, rows)
        err, _ = row_rel_err(full_o[bb, h, rows].cpu().numpy(), ref, den)
        assert err <= TOL_BF16, err
        want = oracle.state(x.k64[bb, h], x.v64[bb, h], n)
        bound = 2.0**-8 * oracle.state(np.abs(x.k64[bb, h]), np.abs(x.v64[bb, h]), n)
        got = np.concatenate([S[bb, h].cpu().numpy(), z[bb, h].cpu().numpy()[:, None]], axis=1)
        assert np.all(np.abs(got - want) <= bound)


def test_reused_and_garbage_workspace():
    # one workspace for calls of different shapes and for arbitrary prior contents: each call's
    # outputs are bit for bit those of a call on a fresh workspace
    import torch

    cfg = _cfg()
    shapes = [(4, 16, 8192), (2, 8, 1500), (4, 16, 8192), (1, 3, 4000)]
    need = max(rs.taylor_prefill_workspace_bytes(cfg, *s) for s in shapes)
    ws = torch.empty((need,), dtype=torch.uint8, device=DEV)
    for fill in (0x00, 0xFF, None):
        announce("single-pass workspace", fill)
        if fill is None:
            ws.random_(0, 256)
        else:
            ws.fill_(fill)
        for i, (B, H, N) in enumerate(shapes):
            x = synth.make_qkv(970 + i, B, H, N, 16, 64, "bf16")
            q, k, v = x.torch(DEV)
            o = torch.empty((B, H, N, 64), device=DEV)
            st = torch.empty((B, H, rs.taylor_state_stride(cfg)), device=DEV)
            rs.taylor_attn_prefill_into(q, k, v, o, None, st, ws, cfg)
            o_ref = torch.empty_like(o)
            st_ref = torch.empty_like(st)
            rs.taylor_attn_prefill_into(q, k, v, o_ref, None, st_ref, rs.new_workspace(cfg, B, H, N, DEV), cfg)
            torch.cuda.synchronize()
            assert torch.equal(o, o_ref) and torch.equal(st, st_ref), f"shape {(B, H, N)} fill {fill}"


def test_graph_replays_interleaved_with_eager_calls():
    # the recorded call clears its flags and uses one tag at every replay; eager calls on the same
    # workspace in between leave flags with their own tags.  Every replay equals the eager result.
    import torch

    B, H, N = 4, 16, 8192
    cfg = _cfg()
    x = synth.make_qkv(980, B, H, N, 16, 64, "bf16")
    q, k, v = x.torch(DEV)
    ws = rs.new_workspace(cfg, B, H, N, DEV)
    o_g = torch.empty((B, H, N, 64), device=DEV)
    st_g = torch.empty((B, H, rs.taylor_state_stride(cfg)), device=DEV)
    announce("single-pass graph")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rs.taylor_attn_prefill_into(q, k, v, o_g, None, st_g, ws, cfg)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rs.taylor_attn_prefill_into(q, k, v, o_g, None, st_g, ws, cfg)
    o_e = torch.empty_like(o_g)
    st_e = torch.empty_like(st_g)
    for r in range(4):
        o_g.fill_(float("nan"))
        st_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rs.taylor_attn_prefill_into(q, k, v, o_e, None, st_e, ws, cfg)  # eager, same workspace
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {r}: outputs differ"
        assert torch.equal(st_g, st_e), f"replay {r}: states differ"
