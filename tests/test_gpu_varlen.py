"""GPU parity of taylor_attn_prefill_varlen (ragged batches packed head-major) against the oracle.

Each sequence is its own causal history, so its outputs and final state are
compared with the float64 oracle run on that sequence alone, at the bars of the
equal-length prefill (1e-5 relative per output row for float32 inputs, 3e-3 for
bfloat16).  Length mixes include empty sequences, single tokens, chunk-boundary
lengths (63, 64, 65) and one long sequence among many short ones.
"""

import numpy as np
import pytest

import oracle
import recurrent_state_amd as rs
import synth
from gpu_util import announce, row_rel_err, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda"
DK, DV = 16, 64
MIX = [1, 63, 64, 65, 500, 0, 1000, 129]


def _cfg(n, dtype):
    return rs.config(n, DK, DV, 64, 1.0, rs.TAYLOR_BF16 if dtype == "bf16" else rs.TAYLOR_F32)


def _packed(x):
    q, k, v = x.torch(DEV)
    return q, k, v, x.torch_cu(DEV)


def _run(q, k, v, cu, cfg, state=None, want_o=True, max_seqlen=None):
    """One ragged prefill through the C ABI; returns the [H, T, d_v] outputs (or None)."""
    import torch

    H, T = k.shape[:2]
    lens = (cu[1:] - cu[:-1]).cpu()
    N = int(lens.max()) if len(lens) else 0
    N = N if max_seqlen is None else max_seqlen
    o = torch.empty((H, T, DV), dtype=torch.float32, device=DEV) if want_o else None
    ws = rs.new_varlen_workspace(cfg, cu.shape[0] - 1, H, N, T, DEV)
    rs.taylor_attn_prefill_varlen(q, k, v, o, state, ws, cu, N, cfg)
    return o


def _check_state(st, b, h, k64, v64, n, dtype, cfg):
    """The final state of (sequence b, head h) against the oracle's sum over the sequence's keys.

    With bfloat16 inputs the two-byte kernel rounds each phi(k_j) to bfloat16 (relative 2^-9)
    before the state product; the bar allows twice that per entry."""
    S, z = rs.state_views(st, cfg)
    got = np.concatenate([S[b, h].cpu().numpy(), z[b, h].cpu().numpy()[:, None]], axis=1)
    full = oracle.state(k64, v64, n)
    if dtype == "bf16":
        bound = 2.0**-8 * oracle.state(np.abs(k64), np.abs(v64), n)
        assert np.all(np.abs(got - full) <= bound + 1e-6 * np.max(np.abs(full), initial=0.0))
    else:
        assert np.max(np.abs(got - full)) <= 1e-5 * np.max(np.abs(full), initial=0.0)


def _check_outputs(o, x, b, n, dtype, label):
    a, e = int(x.cu[b]), int(x.cu[b + 1])
    if e == a:
        return
    qs, ks, vs = x.seq(b)
    got = o[:, a:e].cpu().numpy()
    for h in range(qs.shape[0]):
        ref, den = oracle.truncated_attention(qs[h], ks[h], vs[h], n)
        err, rows = row_rel_err(got[h], ref, den)
        assert rows > 0
        assert err <= tol_for(dtype), f"{label}: sequence {b} head {h}: rel err {err:.3e}"


@pytest.mark.parametrize(
    "n,dtype",
    [(3, "bf16"), (1, "bf16"), (4, "bf16"), (5, "bf16"), (1, "f32"), (2, "f32"), (3, "f32"), (4, "f32"), (5, "f32")],
)
def test_varlen_orders(n, dtype):
    H = 3
    x = synth.make_ragged(70 + n, MIX, H, DK, DV, dtype)
    cfg = _cfg(n, dtype)
    announce("varlen", n, dtype, MIX, H)
    st = rs.new_state(len(MIX), H, cfg, DEV)
    o = _run(*_packed(x), cfg, st)
    for b in range(len(MIX)):
        _check_outputs(o, x, b, n, dtype, "varlen")
        qs, ks, vs = x.seq(b)
        for h in range(H):
            _check_state(st, b, h, ks[h], vs[h], n, dtype, cfg)


@pytest.mark.parametrize("n,dtype", [(3, "bf16"), (3, "f32"), (5, "f32"), (2, "bf16"), (4, "bf16"), (4, "f32")])
def test_varlen_equal_lengths_agree_with_the_batched_call(n, dtype):
    # Equal lengths through the ragged entry point ([H][B*N] layout, cut into token ranges) against
    # taylor_attn_prefill over [B, H, N] (cut into per-sequence segments): the same values up to
    # float32 summation order, and both within the oracle bar.
    import torch

    B, H, N = 3, 2, 700
    x = synth.make_qkv(75, B, H, N, DK, DV, dtype)
    cfg = _cfg(n, dtype)
    announce("varlen-equal", n, dtype, B, H, N)
    q, k, v = x.torch(DEV)
    st = rs.new_state(B, H, cfg, DEV)
    o = torch.empty((B, H, N, DV), device=DEV)
    rs.taylor_attn_prefill(q, k, v, o, st, rs.new_workspace(cfg, B, H, N, DEV), cfg)

    def pack(t):
        return t.permute(1, 0, 2, 3).reshape(H, B * N, t.shape[-1]).contiguous()

    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device=DEV)
    st2 = rs.new_state(B, H, cfg, DEV)
    o2 = _run(pack(q), pack(k), pack(v), cu, cfg, st2)
    err, _ = row_rel_err(o2.cpu().numpy(), pack(o).cpu().numpy())
    assert err <= tol_for(dtype), err
    assert float((st2 - st).abs().max()) <= 1e-5 * float(st.abs().max())
    ref = oracle.batched(oracle.truncated_attention, x.q64, x.k64, x.v64, n)
    err, _ = row_rel_err(o2.cpu().numpy(), pack(torch.from_numpy(ref[0])).numpy(), ref[1].transpose(1, 0, 2))
    assert err <= tol_for(dtype), err


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_resume(dtype):
    # Two ragged calls carrying the states equal one call over the concatenated sequences
    # (states add across chunks, Abstract); some sequences are empty in one of the calls.
    import torch

    n, H = 3, 2
    first, second = [300, 0, 64, 1000, 5], [233, 50, 0, 17, 700]
    x = synth.make_ragged(76, [a + b for a, b in zip(first, second)], H, DK, DV, dtype)
    cfg = _cfg(n, dtype)
    announce("varlen-resume", dtype, first, second)
    q, k, v, _ = _packed(x)
    st = rs.new_state(len(first), H, cfg, DEV)
    outs = []
    for part in (0, 1):
        idx, cu = [], [0]
        for b in range(len(first)):
            lo = int(x.cu[b]) + (first[b] if part else 0)
            hi = lo + (second[b] if part else first[b])
            idx.extend(range(lo, hi))
            cu.append(cu[-1] + hi - lo)
        idx_t = torch.tensor(idx, dtype=torch.long, device=DEV)
        cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
        parts = [t[:, idx_t].contiguous() for t in (q, k, v)]
        outs.append((_run(*parts, cu_t, cfg, st), cu))
    for b in range(len(first)):
        qs, ks, vs = x.seq(b)
        if first[b] + second[b] == 0:
            continue
        got = np.concatenate(
            [outs[p][0][:, outs[p][1][b] : outs[p][1][b + 1]].cpu().numpy() for p in (0, 1)], axis=1)
        for h in range(H):
            ref, den = oracle.truncated_attention(qs[h], ks[h], vs[h], n)
            err, _ = row_rel_err(got[h], ref, den)
            assert err <= tol_for(dtype), f"sequence {b} head {h}: {err:.3e}"
            _check_state(st, b, h, ks[h], vs[h], n, dtype, cfg)


@pytest.mark.parametrize("n,dtype", [(3, "bf16"), (5, "f32"), (4, "bf16")])
def test_varlen_one_long_many_short(n, dtype):
    # Workgroups take equal ranges of the packed token axis: the long sequence spans many ranges
    # (its pieces chain through the scan) while single ranges hold many short sequences.
    lens = [3000] + [17] * 40 + [1, 0, 64]
    H = 2
    x = synth.make_ragged(77, lens, H, DK, DV, dtype)
    cfg = _cfg(n, dtype)
    announce("varlen-long-short", n, dtype, len(lens))
    st = rs.new_state(len(lens), H, cfg, DEV)
    o = _run(*_packed(x), cfg, st)
    for b in (0, 1, 20, 40, 41, 42, 43):
        _check_outputs(o, x, b, n, dtype, "long-short")
        qs, ks, vs = x.seq(b)
        _check_state(st, b, H - 1, ks[H - 1], vs[H - 1], n, dtype, cfg)


def test_varlen_state_only_and_larger_max_seqlen():
    # o = NULL gives the same states; a max_seqlen above the longest sequence changes nothing
    # (the work is planned on the packed token axis).
    import torch

    n, dtype, H = 3, "bf16", 3
    x = synth.make_ragged(78, MIX, H, DK, DV, dtype)
    cfg = _cfg(n, dtype)
    announce("varlen-state-only", MIX)
    args = _packed(x)
    st = rs.new_state(len(MIX), H, cfg, DEV)
    o = _run(*args, cfg, st)
    st2 = rs.new_state(len(MIX), H, cfg, DEV)
    _run(*args, cfg, st2, want_o=False)
    S, z = rs.state_views(st, cfg)
    S2, z2 = rs.state_views(st2, cfg)
    assert torch.allclose(S2, S, rtol=1e-6, atol=1e-6 * float(S.abs().max()))
    assert torch.allclose(z2, z, rtol=1e-6, atol=1e-6 * float(z.abs().max()))
    st3 = rs.new_state(len(MIX), H, cfg, DEV)
    o3 = _run(*args, cfg, st3, max_seqlen=4000)
    assert torch.equal(o3, o)
    assert torch.equal(st3, st)


@pytest.mark.parametrize("n,dtype", [(3, "bf16"), (3, "f32")])
def test_varlen_serving_mix(n, dtype):
    # 32 prompts of 1..4096 tokens (about 65k tokens) over 8 heads: sampled rows of every
    # sequence (first, last and 3 seeded others per head) and the states of 4 sequences.
    H = 8
    lens = synth.ragged_lengths(79, 32, 1, 4096)
    x = synth.make_ragged(79, lens, H, DK, DV, dtype)
    cfg = _cfg(n, dtype)
    announce("varlen-serving", n, dtype, sum(lens), H)
    st = rs.new_state(len(lens), H, cfg, DEV)
    o = _run(*_packed(x), cfg, st).cpu().numpy()
    rng = np.random.default_rng(7900)
    for b, L in enumerate(lens):
        qs, ks, vs = x.seq(b)
        rows = np.unique(np.concatenate([[0, L - 1], rng.integers(0, L, 3)]))
        a = int(x.cu[b])
        for h in range(H):
            ref, den = oracle.truncated_attention_rows(qs[h], ks[h], vs[h], n, rows)
            err, _ = row_rel_err(o[h, a + rows], ref, den)
            assert err <= tol_for(dtype), f"sequence {b} head {h}: {err:.3e}"
    for b in (0, 7, 19, 31):
        qs, ks, vs = x.seq(b)
        _check_state(st, b, 5, ks[5], vs[5], n, dtype, cfg)
