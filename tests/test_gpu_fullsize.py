"""Parity at full workload sizes, in the launch configuration the benchmark times.

* prefill, bfloat16: B=4, H=16, N=8192, n=3 -- every row of four heads, and sampled rows
  (chunk and segment edges plus seeded random rows) of every other head, against the oracle;
  the final state entry by entry;
* decode: 64 sequences x 16 heads, states from a seeded 65,536-token prefix, 1,000 steps
  replayed from a HIP graph -- two heads at every step, every head at the first and the last
  step, against the oracle's direct O(N) evaluation over the whole history;
* order sweep: B=1, H=16, N=16384, float32, n=1..5, unit-norm and raw (scale 1/4) inputs --
  sampled rows of every head (every row of head 0 at n = 3 and 5) against the oracle.
"""

import ctypes

import numpy as np
import pytest

import oracle
import recurrent_state_amd as rs
import synth
from gpu_util import TOL_BF16, TOL_F32, announce, row_rel_err, run_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _sample_rows(N, seed, extra=8):
    edges = [0, 1, 63, 64, 65, 127, 128, 129, N // 2 - 1, N // 2, N - 65, N - 64, N - 2, N - 1]
    rng = np.random.default_rng(seed)
    rows = set(r for r in edges if 0 <= r < N) | set(int(r) for r in rng.integers(0, N, extra))
    return sorted(rows)


FULL_HEADS = ((0, 0), (1, 5), (2, 10), (3, 15))  # (b, h) compared at every row


def test_prefill_bf16_full_size():
    B, H, N = 4, 16, 8192
    x = synth.make_qkv(3, B, H, N, 16, 64, synth.BF16)
    cfg = rs.config(3, 16, 64, 128, 1.0, rs.TAYLOR_BF16)
    announce("full-prefill-bf16", B, H, N)
    st = rs.new_state(B, H, cfg, DEV)
    o, _ = run_prefill(x, cfg, DEV, state=st)
    o = o.cpu().numpy()
    worst = 0.0
    for b in range(B):
        for h in range(H):
            if (b, h) in FULL_HEADS:
                # every row of these heads (the direct O(N^2) oracle, a few seconds per head)
                ref, den = oracle.truncated_attention(x.q64[b, h], x.k64[b, h], x.v64[b, h], 3)
                err, _ = row_rel_err(o[b, h], ref, den)
            else:
                rows = _sample_rows(N, 1000 * b + h)
                ref, den = oracle.truncated_attention_rows(x.q64[b, h], x.k64[b, h], x.v64[b, h], 3, rows)
                err, _ = row_rel_err(o[b, h, rows], ref, den)
            worst = max(worst, err)
    assert worst <= TOL_BF16, worst
    # Final state, entry by entry: the kernel rounds each feature phi_f(k_j) to bfloat16 (relative
    # 2^-9) before the float32 sum over tokens, so |S_fc - ref| <= 2^-9 sum_j |phi_f(k_j)| |v_jc| plus the
    # float32 sum's rounding; the bar is twice the first term (2^-8 sum_j |phi_f(k_j)| |[v_j, 1]_c|,
    # oracle.state of |k|, |v|), a bound per entry, not a fraction of the largest entry (z_0 = N).
    S, z = rs.state_views(st, cfg)
    for b, h in ((0, 0), (3, 15), (2, 9)):
        full = oracle.state(x.k64[b, h], x.v64[b, h], 3)
        bound = 2.0**-8 * oracle.state(np.abs(x.k64[b, h]), np.abs(x.v64[b, h]), 3)
        got = np.concatenate([S[b, h].cpu().numpy(), z[b, h].cpu().numpy()[:, None]], axis=1)
        assert np.all(np.abs(got - full) <= bound), float(np.max(np.abs(got - full) / bound))
    print(f"full-size bf16 prefill: worst sampled row error {worst:.2e}")


def test_decode_full_size_graph():
    import torch

    DB, DH, NP, T = 64, 16, 65536, 1000
    cfg = rs.config(3, 16, 64, 128, 1.0, rs.TAYLOR_F32)
    announce("full-decode", DB, DH, NP, T)
    _, kpre, vpre = synth.device_qkv(4, DB, DH, NP, 16, 64, DEV, need_q=False)
    st = rs.new_state(DB, DH, cfg, DEV)
    rs.taylor_attn_prefill(None, kpre, vpre, None, st, rs.new_workspace(cfg, DB, DH, NP, DEV), cfg)
    dq, dk, dv = synth.device_qkv(4, T, DB * DH, 1, 16, 64, DEV, salt=1)
    dq, dk, dv = (t.view(T, DB, DH, -1) for t in (dq, dk, dv))
    out = torch.empty((T, DB, DH, 64), device=DEV)
    L = rs.lib()
    cp = ctypes.byref(cfg)

    def decode(stream):
        for t in range(T):
            assert L.taylor_attn_decode_step(dq[t].data_ptr(), dk[t].data_ptr(), dv[t].data_ptr(), out[t].data_ptr(),
                                             st.data_ptr(), DB, DH, cp, stream) == 0

    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        decode(torch.cuda.current_stream().cuda_stream)
    g.replay()
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    qh, kh, vh = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    worst = 0.0
    for bh in range(DB * DH):
        b, h = divmod(bh, DH)
        k_hist = np.concatenate([kpre[b, h].cpu().numpy(), kh[:, b, h]]).astype(np.float64)
        v_hist = np.concatenate([vpre[b, h].cpu().numpy(), vh[:, b, h]]).astype(np.float64)
        steps = range(T) if bh in (0, DB * DH - 1) else (0, T - 1)
        for t in steps:
            ref, _ = oracle.decode_reference(qh[t, b, h], k_hist[: NP + t + 1], v_hist[: NP + t + 1], 3)
            err = np.linalg.norm(o[t, b, h] - ref) / np.linalg.norm(ref)
            worst = max(worst, err)
    assert worst <= TOL_F32, worst
    print(f"full-size decode: worst relative error {worst:.2e}")


@pytest.mark.parametrize("unit_norm", [True, False])
def test_order_sweep_full_size(unit_norm):
    B, H, N = 1, 16, 16384
    scale = 1.0 if unit_norm else 0.25
    x = synth.make_qkv(5, B, H, N, 16, 64, synth.F32, unit_norm=unit_norm)
    lines = []
    for n in range(1, 6):
        cfg = rs.config(n, 16, 64, 64, scale, rs.TAYLOR_F32)
        announce("order-sweep", n, "unit" if unit_norm else "raw")
        o, _ = run_prefill(x, cfg, DEV)
        o = o.cpu().numpy()
        worst = 0.0
        for h in range(H):
            if h == 0 and n in (3, 5):
                # every row of one head at the orders the bench leads with and the widest one
                ref, den = oracle.truncated_attention(x.q64[0, h], x.k64[0, h], x.v64[0, h], n, scale)
                err, _ = row_rel_err(o[0, h], ref, den)
            else:
                rows = _sample_rows(N, 77 * h + n, extra=4)
                ref, den = oracle.truncated_attention_rows(x.q64[0, h], x.k64[0, h], x.v64[0, h], n, rows, scale)
                err, _ = row_rel_err(o[0, h, rows], ref, den)
            worst = max(worst, err)
        assert worst <= TOL_F32, (n, worst)
        lines.append(f"n={n}: {worst:.1e}")
    print("order sweep", "unit" if unit_norm else "raw", ", ".join(lines))
