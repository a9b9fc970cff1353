"""Benchmark of the Taylor-attention hot path on one MI355X.

One step = one pass of the whole path:
  * taylor_attn_prefill_into from an empty history (no incoming state array) over one
    batch of B=4 x H=16 x N=8192 bfloat16 tokens (d_k=16, d_v=64, n=3; the kernels walk
    64-token chunks), float32 outputs and final state;
  * 1,000 taylor_attn_decode_step calls on 64 sequences x 16 heads whose float32
    states (153 x 65 per head) were built by a state-only prefill of a seeded
    65,536-token prefix (setup, untimed).  The 1,000 decode launches are replayed
    from one HIP graph (captured once; inputs for all 1,000 steps are resident).
Inputs are seeded synthetic data (synth module): unit-norm Gaussian q, k, Gaussian v.

Reported: prefill tokens/s (B*N / prefill time) as `value`, decode microseconds per
token (per decode step of all 64 sequences), each against its roofline; the oracle's
CPU throughput on a bounded sample of the same prefill workload; and, in `roofline`,
the dominant kernel (the decode step: 1,000 launches per step) measured with HIP
events on the stream it runs on.

Secondary timings after the timed steps (each can be skipped by a flag): decode over
512 sequences whose states exceed the last-level cache, the float32 prefill at
B=1, H=8, N=4,096, n = 3 with its error against exact softmax, the float32 prefill at
n = 1..5 (B=1, H=16, N=16,384) for unit-norm and raw (scale 1/4) inputs with the error of
each order against exact softmax, the expanded-softmax readout (orders 1, 2) on the
main prefill inputs, the backward (gradients of that prefill), a ragged-batch
prefill (32 prompts of seeded lengths 1..2,047, 16 heads, bfloat16, n = 3), and, as
context, exact causal softmax attention (torch's flash kernel) next to the bf16 prefill
at B=4, H=16, N=128..8,192.  Exact softmax for the accuracy figures is evaluated with
float64 torch operations on the device (a comparator, like the flash kernel for time).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tok/s + decode µs/token (n=3,d_k=16,d_v=64), % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3  # MI355X fp32 matrix

# Prefill workload: B=4, H=16, N=8192, bf16 inputs, fp32 states/outputs (the config asks for chunk
# 128; the matrix-core kernels walk 64-token chunks, which the flop count below uses).
PB, PH, PN, DK, DV, NT, PC = 4, 16, 8192, 16, 64, 3, 128
PC_RUN = 64  # chunk the bf16 kernels walk (taylor_prefill_chunk), checked at run time
# Decode workload: 64 sequences x 16 heads, 65,536-token prefix, 1,000 steps.
DB, DH, DPREFIX, DSTEPS = 64, 16, 65536, 1000

W = 153  # feature width at n=3, d_k=16
STATE_BYTES = W * (DV + 1) * 4  # 39,780 B per head
# Algorithmic bytes per decode head-step: state read + written, q, k, v read, o written (fp32).
DECODE_BYTES_PER_HEAD = 2 * STATE_BYTES + 4 * (DK + DK + DV + DV)
# Algorithmic prefill per token-head: q, k, v (bf16) in, o (fp32) out.
PREFILL_BYTES_PER_TOKEN_HEAD = 2 * (DK + DK + DV) + 4 * DV


def prefill_flops_per_token_head(w, chunk):
    """Algorithmic prefill flops per token-head at feature width w and chunk length `chunk` (unpadded
    widths, causal half of each chunk): chunk-state GEMM 2*W*(d_v+1) + readout GEMM 2*W*(d_v+1) +
    intra-chunk scores 2*d_k*(C+1)/2 + intra-chunk PV 2*(d_v+1)*(C+1)/2."""
    return 4 * w * (DV + 1) + DK * (chunk + 1) + (DV + 1) * (chunk + 1)


PREFILL_FLOPS_PER_TOKEN_HEAD = prefill_flops_per_token_head(W, PC_RUN)  # 45,045 at n = 3, C = 64
ABSTRACT_ERROR_N3 = 6.5e-4  # "Expanding Attention", Abstract: error at n = 3 (metric and workload unstated)

DECODE_KERNEL_SOURCE = os.path.join(ROOT, "recurrent_state_amd", "csrc", "decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel_key, source):
    """Per-launch HBM bytes from committed rocprofv3 counters, or None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_sha") != _sha(source):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(x, budget_s=12.0):
    """The float64 oracle on whole heads of the prefill workload until the budget is spent."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    heads = 0
    t0 = time.perf_counter()
    for b in range(PB):
        for h in range(PH):
            oracle.truncated_attention(x.q64[b, h], x.k64[b, h], x.v64[b, h], NT, 1.0)
            heads += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    per_head = dt / heads
    cores = blas_threads or len(os.sched_getaffinity(0))
    return {
        "value": PN / (per_head * PH),  # B*N tokens need B*H heads: (B*N) / (per_head * B*H)
        "unit": "tok/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{heads} of {PB * PH} (b,h) slices of the prefill workload, full N={PN} each, "
                  f"float64 direct O(N^2) oracle, {dt:.1f} s; extrapolated linearly in heads",
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "blas_threads": blas_threads,
    }


def big_decode(rs, synth, torch, dev, seqs=512, steps=100, reps=3, eager=False):
    """Decode with a state set larger than the 256 MB last-level cache (512 sequences x 16 heads:
    326 MB of float32 state), so every step streams the states from HBM.  States come from a
    state-only prefill of a 256-token seeded prefix (the per-step cost does not depend on the
    history length); the steps are replayed from one HIP graph (launched one by one with `eager`).
    Returns a dict for the JSON line."""
    import ctypes

    cfg = rs.config(NT, DK, DV, PC, 1.0, rs.TAYLOR_F32)
    st = rs.new_state(seqs, DH, cfg, dev)
    _, kp, vp = synth.device_qkv(6, seqs, DH, 256, DK, DV, dev, need_q=False)
    rs.taylor_attn_prefill(None, kp, vp, None, st, rs.new_workspace(cfg, seqs, DH, 256, dev), cfg)
    del kp, vp
    q, k, v = synth.device_qkv(6, steps, seqs * DH, 1, DK, DV, dev, salt=1)
    o = torch.empty((steps, seqs * DH, DV), dtype=torch.float32, device=dev)
    f = rs.lib().taylor_attn_decode_step
    cp = ctypes.byref(cfg)

    def run(stream_handle):
        for t in range(steps):
            rc = f(q[t].data_ptr(), k[t].data_ptr(), v[t].data_ptr(), o[t].data_ptr(), st.data_ptr(), seqs, DH, cp,
                   stream_handle)
            if rc:
                raise rs.TaylorError(rc, "taylor_attn_decode_step")

    g = None
    if not eager:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run(torch.cuda.current_stream().cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(torch.cuda.current_stream().cuda_stream)
    else:
        run(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        if g is not None:
            g.replay()
        else:
            run(torch.cuda.current_stream().cuda_stream)
    e1.record()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())
    us = e0.elapsed_time(e1) * 1e3 / (reps * steps)
    nbytes = seqs * DH * DECODE_BYTES_PER_HEAD
    return {"sequences": seqs, "heads": DH, "state_MB": seqs * DH * STATE_BYTES / 1e6, "steps": steps * reps,
            "launch": "eager" if eager else "hip graph of %d steps" % steps,
            "us_per_step": us, "achieved_GBs": nbytes / us / 1e3, "frac_hbm": nbytes / us / 1e3 / HBM_PEAK_GBS}


def softmax_rows(torch, q, k, v, rows, scale):
    """Exact causal softmax attention at the query rows `rows` (a LongTensor) of every (b, h): float64
    torch operations on the device.  q, k: [B, H, N, d_k]; v: [B, H, N, d_v]; returns [B, H, R, d_v]."""
    N = k.shape[2]
    q64 = q[:, :, rows].double()
    k64t = k.double().transpose(-1, -2).contiguous()
    s = scale * torch.matmul(q64, k64t)
    future = torch.arange(N, device=k.device)[None, :] > rows[:, None]
    s = s.masked_fill(future, float("-inf"))
    return torch.matmul(torch.softmax(s, dim=-1), v.double())


def accuracy(o, ref):
    """Error of outputs o against a reference (float64 tensors [..., rows, d_v]) under the three
    metrics reported: max-abs over max |ref|, per-row relative L2 (max and median), relative Frobenius."""
    diff = o.double() - ref
    rr = diff.norm(dim=-1) / ref.norm(dim=-1)
    return {"max_abs_over_max": float(diff.abs().max() / ref.abs().max()), "row_rel_l2_max": float(rr.max()),
            "row_rel_l2_median": float(rr.median()), "rel_frobenius": float(diff.norm() / ref.norm())}


def prefill_into_call(rs, torch, q, k, v, o, state_in, state_out, ws, cfg):
    """A closure making the taylor_attn_prefill_into C-ABI call with fixed raw arguments, for timed loops.
    The binding function is called once first, so its argument checks run; the closure then skips them
    (they cost tens of microseconds of host time per call, as much as the smallest prefills take on the
    GPU, which would otherwise time the host)."""
    import ctypes

    rs.taylor_attn_prefill_into(q, k, v, o, state_in, state_out, ws, cfg)
    B, H, N = k.shape[:3]
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    args = (ptr(q), ptr(k), ptr(v), ptr(o), ptr(state_in), ptr(state_out), ptr(ws), B, H, N, ctypes.byref(cfg),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    f = rs.lib().taylor_attn_prefill_into

    def call():
        rc = f(*args)
        if rc:
            raise rs.TaylorError(rc, "taylor_attn_prefill_into")

    return call


def timed_us(torch, fn, reps):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def order_sweep(rs, synth, torch, dev, reps=3, rows_per_head=256):
    """Prefill at the order-sweep shape (B=1, H=16, N=16,384, float32) for n = 1..5, unit-norm inputs
    (scale 1) and raw ones (q, k ~ N(0, 1) un-normalised, scale 1/sqrt(d_k) = 1/4), timed with HIP
    events (a prefill from an empty history writing the final state, as in the main step).  Algorithmic
    flops per token-head at the chunk the kernels walk.  Accuracy: the outputs at `rows_per_head`
    seeded rows of every head against exact causal softmax on the same inputs (the Abstract: accuracy
    improves exponentially in n for normalised q, k; without normalisation adding terms stops helping)."""
    import numpy as np

    B, H, N = 1, 16, 16384
    rows = np.unique(np.concatenate([[0, 1, 63, 64, N - 1],
                                     np.random.default_rng(55).integers(0, N, rows_per_head - 5)]))
    rows_t = torch.from_numpy(rows).to(dev)
    res = {"rows_per_head": int(len(rows)), "abstract_error_n3": ABSTRACT_ERROR_N3}
    for variant, unit, scale in (("unit_norm", True, 1.0), ("raw_scale_0.25", False, 0.25)):
        x = synth.make_qkv(5, B, H, N, DK, DV, synth.F32, unit_norm=unit)
        q, k, v = x.torch(dev)
        ref = softmax_rows(torch, q, k, v, rows_t, scale)
        o = torch.empty((B, H, N, DV), dtype=torch.float32, device=dev)
        out = {}
        for n in range(1, 6):
            cfg = rs.config(n, DK, DV, 0, scale, rs.TAYLOR_F32)
            chunk = rs.taylor_prefill_chunk(cfg)
            st = torch.empty((B, H, rs.taylor_state_stride(cfg)), dtype=torch.float32, device=dev)
            ws = rs.new_workspace(cfg, B, H, N, dev)
            us = timed_us(torch, prefill_into_call(rs, torch, q, k, v, o, None, st, ws, cfg), reps)
            w = rs.taylor_feature_width(n, DK)
            flops = B * H * N * prefill_flops_per_token_head(w, chunk)
            out[f"n{n}"] = {"W": w, "chunk": chunk, "us": us, "tok_s": B * N / us * 1e6, "TFLOPs": flops / us / 1e6,
                            "frac_fp32_mfma": flops / us / 1e6 / FP32_PEAK_TFLOPS,
                            "error_vs_softmax": accuracy(o[:, :, rows_t], ref)}
            del ws, st
        res[variant] = out
        del x, q, k, v, o, ref
    return res


def prefill_f32_config(rs, synth, torch, dev, reps=20):
    """The float32 prefill workload B=1, H=8, N=4,096, n = 3 (unit-norm q, k; scale 1): a prefill from an
    empty history writing the final state, HIP events; algorithmic flops at the chunk the kernels walk
    against the float32 matrix peak and bytes (q, k, v in, o out, float32) against HBM; and the error of
    every output row against exact causal softmax on the same inputs."""
    B, H, N, n = 1, 8, 4096, 3
    x = synth.make_qkv(2, B, H, N, DK, DV, synth.F32)
    q, k, v = x.torch(dev)
    cfg = rs.config(n, DK, DV, 64, 1.0, rs.TAYLOR_F32)
    chunk = rs.taylor_prefill_chunk(cfg)
    o = torch.empty((B, H, N, DV), dtype=torch.float32, device=dev)
    st = torch.empty((B, H, rs.taylor_state_stride(cfg)), dtype=torch.float32, device=dev)
    ws = rs.new_workspace(cfg, B, H, N, dev)
    us = timed_us(torch, prefill_into_call(rs, torch, q, k, v, o, None, st, ws, cfg), reps)
    w = rs.taylor_feature_width(n, DK)
    flops = B * H * N * prefill_flops_per_token_head(w, chunk)
    nbytes = B * H * N * 4 * (DK + DK + DV + DV)
    ref = softmax_rows(torch, q, k, v, torch.arange(N, device=dev), 1.0)
    return {"workload": f"prefill B{B}xH{H}xN{N} fp32, n={n}, kernel chunk {chunk}", "us": us,
            "tok_s": B * N / us * 1e6, "TFLOPs": flops / us / 1e6, "frac_fp32_mfma": flops / us / 1e6 / FP32_PEAK_TFLOPS,
            "GBs": nbytes / us / 1e3, "frac_hbm": nbytes / us / 1e3 / HBM_PEAK_GBS, "alg_flops": flops,
            "alg_bytes": nbytes, "error_vs_softmax_all_rows": accuracy(o, ref),
            "abstract_error_n3": ABSTRACT_ERROR_N3}


def varlen_prefill(rs, synth, torch, dev, reps=5):
    """Ragged-batch prefill: 32 prompts of 1..2047 seeded lengths (about the main step's 32k tokens per
    head), 16 heads, bfloat16 inputs, n = 3, packed head-major; a prefill from empty histories writing
    the final states, HIP events."""
    H, n = 16, 3
    lens = synth.ragged_lengths(6, 32, 1, 2047)
    x = synth.make_ragged(6, lens, H, DK, DV, synth.BF16)
    q, k, v = x.torch(dev)
    cu = x.torch_cu(dev)
    T, N = sum(lens), max(lens)
    cfg = rs.config(n, DK, DV, 0, 1.0, rs.TAYLOR_BF16)
    o = torch.empty((H, T, DV), dtype=torch.float32, device=dev)
    st = torch.empty((len(lens), H, rs.taylor_state_stride(cfg)), dtype=torch.float32, device=dev)
    ws = rs.new_varlen_workspace(cfg, len(lens), H, N, T, dev)

    def step():
        rs.taylor_attn_prefill_varlen_into(q, k, v, o, None, st, ws, cu, N, cfg)

    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        step()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    return {"sequences": len(lens), "heads": H, "tokens": T, "max_len": N, "us": us, "tok_s": T / us * 1e6}


def centered_prefill(rs, torch, dev, q, k, v, reps=5):
    """The expanded-softmax readout (orders 1, 2) on the main step's prefill inputs (B4 x H16 x N8192,
    bfloat16): a prefill from an empty history writing the final state, HIP events; the states are the
    truncated kernel's of n = order+1."""
    B, H, N = k.shape[:3]
    o = torch.empty((B, H, N, DV), dtype=torch.float32, device=dev)
    res = {}
    for order in (1, 2):
        cfg = rs.config(order + 1, DK, DV, 0, 1.0, rs.TAYLOR_BF16, rs.TAYLOR_READOUT_CENTERED)
        st = torch.empty((B, H, rs.taylor_state_stride(cfg)), dtype=torch.float32, device=dev)
        ws = rs.new_workspace(cfg, B, H, N, dev)

        step = prefill_into_call(rs, torch, q, k, v, o, None, st, ws, cfg)

        step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            step()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        res[f"order{order}"] = {"us": us, "tok_s": B * N / us * 1e6}
        del ws, st
    return res


def backward_prefill(rs, torch, dev, q, k, v, reps=3):
    """taylor_attn_prefill_backward on the main step's prefill inputs (B4 x H16 x N8192, bfloat16, n = 3),
    with outputs from the float32 forward and a seeded upstream gradient; HIP events.  Algorithmic
    flops per token-head (unpadded W = 153), split by the matrix cores that run them with bfloat16
    inputs: on bfloat16 MFMAs (exact products of bfloat16 values) the state updates S += phi(K)^T V of
    the state pass and pass A and pass B's G v, 3 * 2*W*64; on float32 MFMAs pass A's S^T gh and G
    update, pass B's G^T phi(k) and G update, 4 * 2*W*64, the normaliser parts 2*W + 2*W, and the
    intra-chunk products 4*(C+1)/2*(16 + 64) at C = 64.  Each part is reported against its own peak,
    and `frac_mixed_peak` is the time both parts would take at their peaks, back to back, over the
    measured time."""
    B, H, N = k.shape[:3]
    cfg = rs.config(NT, DK, DV, 0, 1.0, rs.TAYLOR_BF16)
    f32 = rs.config(NT, DK, DV, 0, 1.0, rs.TAYLOR_F32)
    o = torch.empty((B, H, N, DV), dtype=torch.float32, device=dev)
    rs.taylor_attn_prefill(q.float(), k.float(), v.float(), o, None, rs.new_workspace(f32, B, H, N, dev), f32)
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    g = torch.randn((B, H, N, DV), generator=gen, device=dev)
    dq = torch.empty((B, H, N, DK), device=dev)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(o)
    ws = rs.new_backward_workspace(cfg, B, H, N, dev)
    rs.taylor_attn_prefill_backward(q, k, v, o, g, None, None, dq, dk, dv, ws, cfg)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        rs.taylor_attn_prefill_backward(q, k, v, o, g, None, None, dq, dk, dv, ws, cfg)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    bf16 = B * H * N * 3 * 2 * W * DV
    fp32 = B * H * N * (4 * 2 * W * DV + 4 * W + 4 * 65 / 2 * (DK + DV))
    floor_us = bf16 / (BF16_PEAK_TFLOPS * 1e6) + fp32 / (FP32_PEAK_TFLOPS * 1e6)
    return {"us": us, "tok_s": B * N / us * 1e6,
            "bf16_mfma": {"alg_flops": bf16, "TFLOPs": bf16 / us / 1e6, "frac_bf16_peak": bf16 / us / 1e6 / BF16_PEAK_TFLOPS},
            "fp32_mfma": {"alg_flops": fp32, "TFLOPs": fp32 / us / 1e6, "frac_fp32_peak": fp32 / us / 1e6 / FP32_PEAK_TFLOPS},
            "floor_us_at_peaks": floor_us, "frac_mixed_peak": floor_us / us}


def backward_flops_per_token_head(w, chunk):
    """Algorithmic flops of the backward per token-head in the factorised form: forward walk S g_i
    (2*W*d_v) and S, z += phi(k)^T [v | 1] (2*W*(d_v + 1)) and the normaliser part (2*W); reverse walk
    G_S^T phi(k_j), G_S v_j (2*W*d_v each) and G += phi(a)^T [gh | -delta] (2*W*(d_v + 1)); intra-chunk
    products over the causal half of a chunk ((C + 1) / 2 keys per query): scores twice (2*d_k each),
    g.v and gh.v (2*d_v each), dv (2*d_v), dq and dk (2*d_k each)."""
    return 2 * w * (5 * DV + 3) + (chunk + 1) / 2 * (8 * DK + 6 * DV)


def backward_orders(rs, synth, torch, dev, reps=2):
    """taylor_attn_prefill_backward at the order-sweep shape (B1 x H16 x N16384, float32, unit-norm q, k)
    for n = 3, 4, 5, with the library's float32 forward outputs and a seeded upstream gradient, HIP events
    around raw C-ABI calls; algorithmic flops (backward_flops_per_token_head at the chunk each kernel
    walks: 64 at n = 3, 32 at n = 4, 5) against the float32 matrix peak, and the time over the forward's."""
    import ctypes

    B, H, N = 1, 16, 16384
    x = synth.make_qkv(5, B, H, N, DK, DV, synth.F32)
    q, k, v = x.torch(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(78)
    g = torch.randn((B, H, N, DV), generator=gen, device=dev)
    o = torch.empty((B, H, N, DV), dtype=torch.float32, device=dev)
    dq = torch.empty((B, H, N, DK), device=dev)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(o)
    res = {}
    for n in (3, 4, 5):
        cfg = rs.config(n, DK, DV, 0, 1.0, rs.TAYLOR_F32)
        fwd = prefill_into_call(rs, torch, q, k, v, o, None, None, rs.new_workspace(cfg, B, H, N, dev), cfg)
        fwd_us = timed_us(torch, fwd, reps)
        ws = rs.new_backward_workspace(cfg, B, H, N, dev)
        rs.taylor_attn_prefill_backward(q, k, v, o, g, None, None, dq, dk, dv, ws, cfg)
        ptr = lambda t: ctypes.c_void_p(t.data_ptr())
        args = (ptr(q), ptr(k), ptr(v), ptr(o), ptr(g), None, None, ptr(dq), ptr(dk), ptr(dv),
                None if ws is None else ptr(ws), B, H, N, ctypes.byref(cfg),
                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        f = rs.lib().taylor_attn_prefill_backward

        def call():
            rc = f(*args)
            if rc:
                raise rs.TaylorError(rc, "taylor_attn_prefill_backward")

        us = timed_us(torch, call, reps)
        w = rs.taylor_feature_width(n, DK)
        chunk = 64 if n <= 3 else 32
        flops = B * H * N * backward_flops_per_token_head(w, chunk)
        res["n%d" % n] = {"W": w, "chunk": chunk, "us": us, "tok_s": B * N / us * 1e6, "forward_us": fwd_us,
                          "over_forward": us / fwd_us, "alg_flops": flops, "TFLOPs": flops / us / 1e6,
                          "frac_fp32_mfma": flops / us / 1e6 / FP32_PEAK_TFLOPS,
                          "workspace_MB": (0 if ws is None else ws.numel()) / 1e6}
        del ws
        torch.cuda.empty_cache()
    return res


def softmax_crossover(rs, synth, torch, dev, reps=5):
    """Context: exact causal softmax attention (torch's fused flash kernel, bfloat16, scale 1) against the
    bfloat16 prefill (n = 3, from an empty history, final state written) at B = 4, H = 16 for N = 128 ..
    8192, both timed with HIP events.  The flash kernel takes equal head widths, so q and k are padded
    with zero columns to d_v = 64 (the scores are unchanged).  Only the flash and memory-efficient
    backends are allowed; if neither runs, the error is reported instead of a time."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import torch.nn.functional as F
    B, H = 4, 16
    cfg = rs.config(NT, DK, DV, 0, 1.0, rs.TAYLOR_BF16)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    res, backend, crossover = {}, None, None
    for N in (128, 256, 512, 1024, 2048, 4096, 8192):
        x = synth.make_qkv(3, B, H, N, DK, DV, synth.BF16)
        q, k, v = x.torch(dev)
        o = torch.empty((B, H, N, DV), dtype=torch.float32, device=dev)
        st = torch.empty((B, H, rs.taylor_state_stride(cfg)), dtype=torch.float32, device=dev)
        ws = rs.new_workspace(cfg, B, H, N, dev)
        t_us = timed(prefill_into_call(rs, torch, q, k, v, o, None, st, ws, cfg))
        qp = torch.nn.functional.pad(q, (0, DV - DK)).contiguous()
        kp = torch.nn.functional.pad(k, (0, DV - DK)).contiguous()
        s_us, err = None, None
        for be in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
            try:
                with sdpa_kernel([be]):
                    s_us = timed(lambda: F.scaled_dot_product_attention(qp, kp, v, is_causal=True, scale=1.0))
                backend = str(be).split(".")[-1]
                break
            except RuntimeError as e:
                err = str(e).splitlines()[0][:200]
        row = {"taylor_us": t_us, "softmax_us": s_us}
        if s_us is None:
            row["softmax_error"] = err
        else:
            row["softmax_over_taylor"] = s_us / t_us
        res[f"N{N}"] = row
        del x, q, k, v, o, st, ws, qp, kp
    # the smallest N from which the prefill is faster at every larger N of the sweep
    for key in sorted((kk for kk in res if kk.startswith("N")), key=lambda kk: -int(kk[1:])):
        if res[key].get("softmax_over_taylor", 0.0) <= 1.0:
            break
        crossover = int(key[1:])
    res["softmax_backend"] = backend
    res["prefill_faster_from_N"] = crossover
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=DSTEPS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager-decode", action="store_true", help="launch decode steps one by one (no graph)")
    ap.add_argument("--no-big-decode", action="store_true",
                    help="skip the secondary decode run whose states exceed the last-level cache")
    ap.add_argument("--big-decode-steps", type=int, default=100)
    ap.add_argument("--no-order-sweep", action="store_true", help="skip the n = 1..5 float32 prefill timings")
    ap.add_argument("--no-f32-config", action="store_true",
                    help="skip the float32 B1 x H8 x N4096 prefill and its error against softmax")
    ap.add_argument("--no-varlen", action="store_true", help="skip the ragged-batch prefill timing")
    ap.add_argument("--no-centered", action="store_true", help="skip the expanded-softmax readout timing")
    ap.add_argument("--no-softmax", action="store_true", help="skip the exact softmax attention comparison")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-backward-orders", action="store_true", help="skip the backward timing at n = 3, 4, 5")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 3 times (scale reference for "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch

        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "copies": 3}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path is data-parallel "
              f"over (batch, head); see the sharding notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    import recurrent_state_amd as rs
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = rs.lib()
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)

    # ---- prefill workload ----
    x = synth.make_qkv(3, PB, PH, PN, DK, DV, synth.BF16)
    pq, pk, pv = x.torch(dev)
    pcfg = rs.config(NT, DK, DV, PC, 1.0, rs.TAYLOR_BF16)
    po = torch.empty((PB, PH, PN, DV), dtype=torch.float32, device=dev)
    pstate = torch.empty((PB, PH, rs.taylor_state_stride(pcfg)), dtype=torch.float32, device=dev)
    pws = rs.new_workspace(pcfg, PB, PH, PN, dev)
    if rs.taylor_prefill_chunk(pcfg) != PC_RUN:
        raise RuntimeError(f"the bf16 prefill walks {rs.taylor_prefill_chunk(pcfg)}-token chunks, the flop count assumes {PC_RUN}")
    log("prefill inputs ready")

    # ---- decode workload: states from a 65,536-token prefix ----
    dcfg = rs.config(NT, DK, DV, PC, 1.0, rs.TAYLOR_F32)
    dstate = rs.new_state(DB, DH, dcfg, dev)
    _, kpre, vpre = synth.device_qkv(4, DB, DH, DPREFIX, DK, DV, dev, need_q=False)
    ws = rs.new_workspace(dcfg, DB, DH, DPREFIX, dev)
    rs.taylor_attn_prefill(None, kpre, vpre, None, dstate, ws, dcfg)
    torch.cuda.synchronize()
    del kpre, vpre, ws
    torch.cuda.empty_cache()
    T = args.decode_steps
    dq, dk_, dv_ = synth.device_qkv(4, T, DB * DH, 1, DK, DV, dev, salt=1)
    dq, dk_, dv_ = (t.view(T, DB, DH, -1) for t in (dq, dk_, dv_))
    dout = torch.empty((T, DB, DH, DV), dtype=torch.float32, device=dev)
    log("decode states and inputs ready")

    cfgp = __import__("ctypes").byref(dcfg)

    def decode_all(stream_handle):
        f = lib.taylor_attn_decode_step
        qp, kp, vp, op, sp = dq.data_ptr(), dk_.data_ptr(), dv_.data_ptr(), dout.data_ptr(), dstate.data_ptr()
        qs, vs = DB * DH * DK * 4, DB * DH * DV * 4
        for t in range(T):
            rc = f(qp + t * qs, kp + t * qs, vp + t * vs, op + t * vs, sp, DB, DH, cfgp, stream_handle)
            if rc:
                raise rs.TaylorError(rc, "taylor_attn_decode_step")

    graph = None
    if not args.eager_decode:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            decode_all(torch.cuda.current_stream().cuda_stream)  # warm-up outside capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decode_all(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        log("decode graph captured")

    prefill_step = prefill_into_call(rs, torch, pq, pk, pv, po, None, pstate, pws, pcfg)

    def step(evs):
        cur = torch.cuda.current_stream()
        evs[0].record(cur)
        prefill_step()
        evs[1].record(cur)
        if graph is not None:
            graph.replay()
        else:
            decode_all(cur.cuda_stream)
        evs[2].record(cur)

    for _ in range(args.warmup):
        step([torch.cuda.Event(enable_timing=True) for _ in range(3)])
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pre_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    step_ms = sum(e[0].elapsed_time(e[2]) for e in events) / args.steps
    assert bool(torch.isfinite(po).all()) and bool(torch.isfinite(dout).all())

    decode_launch_s = dec_ms / 1e3 / T
    decode_bytes = DB * DH * DECODE_BYTES_PER_HEAD
    dec_gbs = decode_bytes / decode_launch_s / 1e9
    prefill_s = pre_ms / 1e3
    prefill_tok_s = PB * PN / prefill_s
    p_bytes = PB * PH * PN * PREFILL_BYTES_PER_TOKEN_HEAD
    p_flops = PB * PH * PN * PREFILL_FLOPS_PER_TOKEN_HEAD
    traffic = measured_traffic("decode_step", DECODE_KERNEL_SOURCE)

    out = {
        "metric": METRIC,
        "value": prefill_tok_s,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded unit-norm Gaussian q,k; Gaussian v)",
        "config": {
            "workload": f"prefill B{PB}xH{PH}xN{PN} bf16 in, fp32 state/out, kernel chunk {PC_RUN}; "
                        f"decode {DB} seq x {DH} heads, fp32 state, {DPREFIX}-token prefix, {T} steps/step",
            "n_terms": NT, "d_k": DK, "d_v": DV, "global_batch": PB, "seq_len": PN,
            "parallelism": "none (1 GPU)",
        },
        "decode_us_per_token": dec_ms * 1e3 / T,
        "decode_tokens_per_s": DB * T / (dec_ms / 1e3),
        "decode_launch": "hip graph of %d steps" % T if graph is not None else "eager",
        "prefill_ms": pre_ms,
        "prefill": {
            "bound": "hbm", "achieved_GBs": p_bytes / prefill_s / 1e9, "peak_GBs": HBM_PEAK_GBS,
            "frac_hbm": p_bytes / prefill_s / 1e9 / HBM_PEAK_GBS,
            "achieved_TFLOPs": p_flops / prefill_s / 1e12, "bf16_peak_TFLOPs": BF16_PEAK_TFLOPS,
            "frac_bf16_mfma": p_flops / prefill_s / 1e12 / BF16_PEAK_TFLOPS,
            "alg_bytes": p_bytes, "alg_flops": p_flops, "chunk": PC_RUN,
            # attainable roofline min(peak_MFMA, AI * BW): the larger of the HBM and matrix-core floors
            "floor_us": max(p_bytes / (HBM_PEAK_GBS * 1e3), p_flops / (BF16_PEAK_TFLOPS * 1e6)),
            "frac_attainable": max(p_bytes / (HBM_PEAK_GBS * 1e3), p_flops / (BF16_PEAK_TFLOPS * 1e6)) / (prefill_s * 1e6),
        },
        "roofline": {
            "kernel": "decode_kernel<3,16,64,float>",
            "bound": "hbm",
            "achieved": dec_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": dec_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "alg_bytes_per_launch": decode_bytes,
            "avg_launch_us": decode_launch_s * 1e6,
        },
        "wall_s_timed": wall,
    }
    if not args.no_big_decode:
        log("decode with states above the last-level cache")
        del dq, dk_, dv_, dout, graph
        torch.cuda.empty_cache()
        out["decode_llc_defeating"] = big_decode(rs, synth, torch, dev, steps=args.big_decode_steps,
                                                 eager=args.eager_decode)
    if not args.no_f32_config:
        log("float32 prefill B1 H8 N4096 and its error against exact softmax")
        out["prefill_f32_B1xH8xN4096"] = prefill_f32_config(rs, synth, torch, dev)
    if not args.no_order_sweep:
        log("order sweep n = 1..5 (float32 prefill, B1 H16 N16384, unit-norm and raw) with errors against softmax")
        out["order_sweep_prefill_f32_B1xH16xN16384"] = order_sweep(rs, synth, torch, dev)
    if not args.no_centered:
        log("expanded-softmax readout (orders 1, 2) on the prefill inputs")
        out["prefill_centered_bf16_B4xH16xN8192"] = centered_prefill(rs, torch, dev, pq, pk, pv)
    if not args.no_backward:
        log("backward (gradients of the prefill)")
        out["backward_bf16_B4xH16xN8192"] = backward_prefill(rs, torch, dev, pq, pk, pv)
    if not args.no_backward_orders:
        log("backward at n = 3, 4, 5 (float32, B1 H16 N16384)")
        out["backward_f32_B1xH16xN16384"] = backward_orders(rs, synth, torch, dev)
    if not args.no_varlen:
        log("ragged-batch prefill (32 prompts, 16 heads, bf16)")
        out["prefill_varlen_bf16_32seqs_H16"] = varlen_prefill(rs, synth, torch, dev)
    if not args.no_softmax:
        log("exact softmax attention (flash kernel) against the prefill, N = 128 .. 8192")
        out["softmax_vs_prefill_bf16_B4xH16"] = softmax_crossover(rs, synth, torch, dev)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
