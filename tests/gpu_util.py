"""Helpers shared by the GPU parity tests (comparison metrics, runners, case announcements)."""

import sys

import numpy as np

import recurrent_state_amd as rs

TOL_F32 = 1e-5  # relative, per output row, float32 inputs
TOL_BF16 = 3e-3  # relative, per output row, bfloat16 inputs (oracle sees the same rounded inputs)
# Float32 rounding allowance per row where a result is a small difference of large terms: 64 unit
# roundoffs (2^-24 each) times the norm of the row's term magnitudes (sums of absolute values of the
# terms, oracle.attention_backward_magnitudes).  64 covers the depth of the kernels' summation trees
# (log2 of 8192 tokens, plus the 4- and 16-deep matrix-core sums) and the roundings that form one term.
ROUND_F32 = 2.0**-18


def announce(*parts):
    """Name the case on stdout before a GPU step (visible even if the step takes the process down)."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def row_rel_err(o, ref, den=None, den_floor=1e-6):
    """max over rows of ||o_i - ref_i||_2 / ||ref_i||_2, skipping rows whose |den| < den_floor * max|den|.

    Returns (error, rows compared).  Odd n never skips (its kernel is positive).
    """
    o = np.asarray(o, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    keep = np.ones(len(ref), dtype=bool)
    if den is not None:
        den = np.abs(np.asarray(den, dtype=np.float64).reshape(-1))
        keep = den >= den_floor * den.max()
    assert np.all(np.isfinite(o[keep])), "non-finite outputs"
    num = np.linalg.norm(o[keep] - ref[keep], axis=1)
    nrm = np.linalg.norm(ref[keep], axis=1)
    return float(np.max(num / nrm)) if keep.any() else 0.0, int(keep.sum())


def rows_within(got, ref, mag, tol):
    """max over rows i of ||got_i - ref_i|| / max(tol ||ref_i||, ROUND_F32 ||mag_i||): at most 1 passes.

    Rows are the last axis.  A row whose reference and magnitudes both vanish must be exactly zero."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(got.shape)
    mag = np.asarray(mag, dtype=np.float64).reshape(got.shape)
    assert np.all(np.isfinite(got)), "non-finite values"
    err = np.linalg.norm(got - ref, axis=1)
    bar = np.maximum(tol * np.linalg.norm(ref, axis=1), ROUND_F32 * np.linalg.norm(mag, axis=1))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bar > 0, err / np.where(bar > 0, bar, 1.0), np.where(err > 0, np.inf, 0.0))
    return float(np.max(ratio)) if len(ratio) else 0.0


def tol_for(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_F32


def run_prefill(x, cfg, device, state=None, want_o=True, stream=None):
    """Prefill through the C ABI on device tensors made from a synth.QKV; returns (o tensor or None, state)."""
    import torch

    q, k, v = x.torch(device)
    B, H, N = k.shape[:3]
    o = torch.empty((B, H, N, cfg.d_v), dtype=torch.float32, device=device) if want_o else None
    ws = rs.new_workspace(cfg, B, H, N, device)
    rs.taylor_attn_prefill(q, k, v, o, state, ws, cfg, stream)
    return o, state
