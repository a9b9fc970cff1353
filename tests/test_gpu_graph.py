"""HIP-graph replay of the library's launches (the benchmark replays decode steps from a graph).

A captured sequence of decode steps (and a captured prefill) is replayed several times with
eager work and synchronisation between replays; every replay must reproduce, bit for bit,
the same calls made eagerly on an identical copy of the state.
"""

import ctypes

import numpy as np
import pytest

import recurrent_state_amd as rs
import synth
from gpu_util import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_decode_graph_replays_match_eager():
    import torch

    B, H, T, N0 = 4, 16, 20, 500
    cfg = rs.config(3, 16, 64, 64)
    announce("graph-decode", B, H, T)
    x = synth.make_qkv(110, B, H, N0, 16, 64)
    q0, k0, v0 = x.torch(DEV)
    st_eager = rs.new_state(B, H, cfg, DEV)
    rs.taylor_attn_prefill(None, k0, v0, None, st_eager, rs.new_workspace(cfg, B, H, N0, DEV), cfg)
    st_graph = st_eager.clone()
    rounds = 3
    steps = [synth.device_qkv(111, T, B * H, 1, 16, 64, DEV, salt=r) for r in range(rounds)]
    sq = torch.empty((T, B, H, 16), device=DEV)
    sk = torch.empty_like(sq)
    sv = torch.empty((T, B, H, 64), device=DEV)
    so = torch.empty((T, B, H, 64), device=DEV)
    L = rs.lib()
    cp = ctypes.byref(cfg)

    def decode(qb, kb, vb, ob, st, stream):
        for t in range(T):
            rc = L.taylor_attn_decode_step(qb[t].data_ptr(), kb[t].data_ptr(), vb[t].data_ptr(), ob[t].data_ptr(),
                                           st.data_ptr(), B, H, cp, stream)
            assert rc == 0

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        decode(sq, sk, sv, so, st_graph, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for r in range(rounds):
        qd, kd, vd = (t.view(T, B, H, -1) for t in steps[r])
        sq.copy_(qd)
        sk.copy_(kd)
        sv.copy_(vd)
        _ = (sq * 2).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        eager_o = torch.empty_like(so)
        decode(qd, kd, vd, eager_o, st_eager, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        a = so.cpu().numpy()
        b = eager_o.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"replay {r} differs"
        assert torch.equal(st_graph, st_eager), f"state after replay {r} differs"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_graph_replays_match_eager(dtype):
    import torch

    B, H, N = 2, 4, 777
    cfg = rs.config(3, 16, 64, 64, 1.0, rs.TAYLOR_BF16 if dtype == "bf16" else rs.TAYLOR_F32)
    announce("graph-prefill", dtype)
    x = synth.make_qkv(112, B, H, N, 16, 64, dtype)
    q, k, v = x.torch(DEV)
    ws = rs.new_workspace(cfg, B, H, N, DEV)
    o_g = torch.empty((B, H, N, 64), device=DEV)
    st_g = torch.empty((B, H, rs.taylor_state_stride(cfg)), device=DEV)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        rs.taylor_state_init(st_g, cfg)
        rs.taylor_attn_prefill(q, k, v, o_g, st_g, ws, cfg)
    o_e = torch.empty_like(o_g)
    st_e = torch.empty_like(st_g)
    for r in range(3):
        o_g.fill_(float("nan"))
        st_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        rs.taylor_state_init(st_e, cfg)
        rs.taylor_attn_prefill(q, k, v, o_e, st_e, rs.new_workspace(cfg, B, H, N, DEV), cfg)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {r}: outputs differ"
        assert torch.equal(st_g, st_e), f"replay {r}: states differ"
