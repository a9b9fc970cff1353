"""Truncated-kernel causal attention, its recurrent form, and causal softmax (oracle; test infrastructure only).

Source: "Expanding Attention: A Taylor-Series Route to Linear-Time Transformers
with a Fixed Number of Recurrent States" (Huang, arXiv:2610.20637), Abstract.

The definition (what the library must reproduce up to rounding order).  Per
(batch, head), with score scale sigma and n Taylor terms:

    s_ij   = sigma * (q_i . k_j)
    K_n(s) = sum_{m=0}^{n-1} s^m / m!                    (the truncated kernel)
    o_i    = sum_{j<=i} K_n(s_ij) v_j / sum_{j<=i} K_n(s_ij)

``truncated_attention`` writes this out directly in O(N^2), blocked by rows of
queries only (no other blocking, fusion or reordering).

Readings taken where the pages are silent (listed again in the design notes):

* causality is inclusive (j <= i), so o_0 = v_0;
* the ratio is taken as is: no epsilon, no clamp, no max-subtraction (the
  truncated kernel needs none; for odd n it is positive for every real s);
* sigma multiplies the score (equivalently q before the feature map).

The remaining routines are separate statements used only to pin the pages'
claims against the definition:

* ``state``/``chunked_state``: the recurrent state sum_j phi(k_j) [v_j, 1]^T
  and its sum over chunks (the Abstract's chunk additivity);
* ``recurrent``: one rank-one update then one readout per token (the
  Abstract's recursion, "lossless with respect to the truncated kernel");
* ``softmax_attention``: exact causal softmax attention, the accuracy reference
  the truncated kernel converges to as n grows (the Abstract's "accuracy
  improves exponentially in n").
"""

import numpy as np

from .features import features


def truncated_kernel(s, n):
    """K_n(s) = sum_{m=0}^{n-1} s^m/m!, evaluated by Horner's rule in float64."""
    s = np.asarray(s, dtype=np.float64)
    acc = np.ones_like(s)
    for m in range(n - 1, 0, -1):
        acc = 1.0 + acc * s / m
    return acc


def truncated_attention(q, k, v, n, scale=1.0, block=512):
    """Direct causal truncated-kernel attention for one head.

    q, k: [N, d_k]; v: [N, d_v].  Returns (o [N, d_v], den [N]) in float64,
    where den_i = sum_{j<=i} K_n(s_ij) is the normaliser.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N = q.shape[0]
    o = np.empty((N, v.shape[1]), dtype=np.float64)
    den = np.empty(N, dtype=np.float64)
    for i0 in range(0, N, block):
        i1 = min(N, i0 + block)
        s = scale * (q[i0:i1] @ k[:i1].T)
        w = truncated_kernel(s, n)
        rows = np.arange(i0, i1)[:, None]
        cols = np.arange(i1)[None, :]
        w[cols > rows] = 0.0
        num = w @ v[:i1]
        den[i0:i1] = w.sum(axis=1)
        o[i0:i1] = num / den[i0:i1, None]
    return o, den


def truncated_attention_rows(q, k, v, n, rows, scale=1.0):
    """The same definition evaluated only at the query rows ``rows`` (any order).

    Row i sees keys 0..i.  Cost O(len(rows) * N); used for sampled checks at
    sizes where the full O(N^2) pass is too slow.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((len(rows), v.shape[1]), dtype=np.float64)
    den = np.empty(len(rows), dtype=np.float64)
    for r, i in enumerate(rows):
        w = truncated_kernel(scale * (k[: i + 1] @ q[i]), n)
        den[r] = w.sum()
        o[r] = (w @ v[: i + 1]) / den[r]
    return o, den


def decode_reference(q_t, k_hist, v_hist, n, scale=1.0):
    """Output of one decode step: the query q_t attends to every key given (inclusive).

    k_hist, v_hist hold the whole history including the current token.
    Returns (o_t [d_v], den_t).  O(N) per step, straight from the definition.
    """
    k_hist = np.asarray(k_hist, dtype=np.float64)
    v_hist = np.asarray(v_hist, dtype=np.float64)
    w = truncated_kernel(scale * (k_hist @ np.asarray(q_t, dtype=np.float64)), n)
    den = w.sum()
    return (w @ v_hist) / den, den


def softmax_attention(q, k, v, scale=1.0, block=512):
    """Exact causal softmax attention for one head, float64: softmax_j(s_ij) over j <= i."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N = q.shape[0]
    o = np.empty((N, v.shape[1]), dtype=np.float64)
    for i0 in range(0, N, block):
        i1 = min(N, i0 + block)
        s = scale * (q[i0:i1] @ k[:i1].T)
        rows = np.arange(i0, i1)[:, None]
        cols = np.arange(i1)[None, :]
        s[cols > rows] = -np.inf
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        o[i0:i1] = (e @ v[:i1]) / e.sum(axis=1, keepdims=True)
    return o


def softmax_attention_rows(q, k, v, rows, scale=1.0):
    """Exact causal softmax attention at the query rows ``rows`` only (row i sees keys 0..i); float64.

    O(len(rows) * N), for accuracy figures at sizes where the full pass is too slow."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((len(rows), v.shape[1]), dtype=np.float64)
    for r, i in enumerate(rows):
        s = scale * (k[: i + 1] @ q[i])
        e = np.exp(s - s.max())
        o[r] = (e @ v[: i + 1]) / e.sum()
    return o


def state(k, v, n):
    """Recurrent state sum_j phi(k_j) [v_j, 1]^T: [W, d_v + 1] float64.

    Columns 0..d_v-1 hold S = sum_j phi(k_j) v_j^T; column d_v holds the
    normaliser z = sum_j phi(k_j).
    """
    phi = features(k, n)
    v1 = np.concatenate([np.asarray(v, dtype=np.float64), np.ones((phi.shape[0], 1))], axis=1)
    return phi.T @ v1


def chunked_state(k, v, n, chunk):
    """Sum over consecutive chunks of ``chunk`` tokens of each chunk's own state."""
    N = np.asarray(k).shape[0]
    total = None
    for c0 in range(0, N, chunk):
        part = state(k[c0 : c0 + chunk], v[c0 : c0 + chunk], n)
        total = part if total is None else total + part
    return total


def recurrent(q, k, v, n, scale=1.0, state0=None):
    """Token-by-token recursion: S += phi(k_t) [v_t, 1]^T, then o_t = (phi(sigma q_t)^T S)[:d_v] / (...)[d_v].

    Returns (o [N, d_v], final state [W, d_v+1]).  ``state0`` continues a
    previous call (the state is the whole memory of the prefix).
    """
    q = np.asarray(q, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    fk = features(k, n)
    fq = features(scale * q, n)
    N, dv = v.shape
    S = np.zeros((fk.shape[1], dv + 1)) if state0 is None else np.array(state0, dtype=np.float64)
    v1 = np.concatenate([v, np.ones((N, 1))], axis=1)
    o = np.empty((N, dv))
    for t in range(N):
        S += np.outer(fk[t], v1[t])
        r = fq[t] @ S
        o[t] = r[:dv] / r[dv]
    return o, S


def batched(fn, q, k, v, *args, **kwargs):
    """Apply a per-head routine over leading [B, H] dims; returns a tuple of stacked results."""
    B, H = q.shape[:2]
    outs = None
    for b in range(B):
        for h in range(H):
            r = fn(q[b, h], k[b, h], v[b, h], *args, **kwargs)
            if not isinstance(r, tuple):
                r = (r,)
            if outs is None:
                outs = [np.empty((B, H) + np.shape(x), dtype=np.float64) for x in r]
            for dst, x in zip(outs, r):
                dst[b, h] = x
    return tuple(outs)
