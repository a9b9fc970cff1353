"""Softmax expanded about the mean score, as causal linear attention (oracle; test infrastructure only).

Source: Su Jianlin, kexue.fm translation 11814 (Taylor expansions of logsumexp
and softmax): "Some Notations" (x-bar is the mean of a vector's components),
"Basic Expansion" (logsumexp of x expanded in y = x - mean(x)), "Calculating the
Gradient" (softmax as the gradient of logsumexp, giving the softmax expansion in
y, whose truncations still sum to one but may go negative) and "Linear
Attention" (the first- and second-order truncations applied to the scores
x_j = q . k_j; the square (q . (k_j - k-bar))^2 is an inner product of outer
products, so the whole expansion is linear attention).

The definition (what the library must reproduce up to rounding order).  For a
score vector x of length n, with y = x - mean(x):

    order 1:  p = (1 + y) / n
    order 2:  p = (1 + y + (y^2 - mean(y^2)) / 2) / n

Causal attention applies it row by row to the prefix: row i has the scores
x_j = sigma * (q_i . k_j) for j <= i (so n = i + 1 and the mean key is the mean
of k_0 .. k_i) and outputs o_i = sum_{j<=i} p_j v_j.  ``centered_attention``
writes this out directly in O(N^2).

Readings taken where the page is silent (listed again in the design notes):

* the page expands the softmax over a full set of n keys; for causal attention
  each query uses the keys j <= i (inclusive), so n and the mean key grow with i;
* sigma multiplies the score, as for the truncated-kernel method;
* no renormalisation and no clamp: the weights sum to one by construction and
  may be negative, and the output is the plain weighted sum.

``lse_series`` is a separate statement of the "Basic Expansion" used only to pin
the weights: their expansion is the gradient of it ("Calculating the Gradient").
"""

import numpy as np


def centered_weights(x, order):
    """Softmax of the last axis of x expanded about its mean and truncated at `order` (1 or 2)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    y = x - x.mean(axis=-1, keepdims=True)
    p = 1.0 + y
    if order >= 2:
        y2 = y * y
        p = p + 0.5 * (y2 - y2.mean(axis=-1, keepdims=True))
    if order not in (1, 2):
        raise ValueError("order must be 1 or 2")
    return p / n


def centered_attention(q, k, v, order, scale=1.0):
    """Causal attention with the expanded softmax, one head: o [N, d_v] float64 (row i sees keys 0..i)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N = q.shape[0]
    o = np.empty((N, v.shape[1]), dtype=np.float64)
    for i in range(N):
        p = centered_weights(scale * (k[: i + 1] @ q[i]), order)
        o[i] = p @ v[: i + 1]
    return o


def centered_attention_rows(q, k, v, order, rows, scale=1.0):
    """The same definition at the query rows ``rows`` only (sampled checks at large N)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((len(rows), v.shape[1]), dtype=np.float64)
    for r, i in enumerate(rows):
        o[r] = centered_weights(scale * (k[: i + 1] @ q[i]), order) @ v[: i + 1]
    return o


def centered_magnitudes(q, k, v, order, scale=1.0):
    """Per-element magnitudes [N, d_v] of the sums behind ``centered_attention``; float64.

    Expanding the centred powers writes row i's weights as p_ij = g0 + g1 s_ij + g2 s_ij^2 / 2 with
    coefficients from the prefix sums c = i + 1, d1 = sum_j s_ij, d2 = sum_j s_ij^2 / 2 and u = d1 / c:
    order 1 g = ((1 - u) / c, 1 / c), order 2 g = ((1 - u + u^2 - d2 / c) / c, (1 - u) / c, 1 / c).
    The magnitudes replace every factor there by its absolute value (s by s_bar = |sigma| |q_i| . |k_j|,
    u by sum_j s_bar_ij / c, d2 by sum_j s_bar_ij^2 / 2, the differences in g by sums) and give
    g0_bar sum_j |v_j| + g1_bar sum_j s_bar_ij |v_j| + g2_bar sum_j s_bar_ij^2 / 2 |v_j|: at least the
    absolute values of the terms a float32 evaluation of this form adds up, in any order.  Not a
    result to reproduce: the bound GPU tests scale their per-row bars by."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if order not in (1, 2):
        raise ValueError("order must be 1 or 2")
    N = q.shape[0]
    out = np.empty((N, v.shape[1]), dtype=np.float64)
    for i in range(N):
        c = i + 1.0
        sb = abs(scale) * (np.abs(k[: i + 1]) @ np.abs(q[i]))
        av = np.abs(v[: i + 1])
        ub = sb.sum() / c
        if order == 1:
            g0, g1, g2 = (1.0 + ub) / c, 1.0 / c, 0.0
        else:
            g0 = (1.0 + ub + ub * ub + 0.5 * (sb * sb).sum() / c) / c
            g1, g2 = (1.0 + ub) / c, 1.0 / c
        out[i] = g0 * av.sum(axis=0) + g1 * (sb @ av) + g2 * (0.5 * sb * sb) @ av
    return out


def lse_series(x, top):
    """logsumexp of the last axis expanded in y = x - mean(x) ("Basic Expansion"), keeping the terms in
    y^2 (top = 2) or y^2 and y^3 (top = 3): log n + mean(x) + mean(y^2)/2 [+ mean(y^3)/6].

    Through y^3 the log(1 + t) step adds nothing (its t^2 term starts at y^4), so these are the
    page's series cut after the named power."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    xm = x.mean(axis=-1)
    y = x - xm[..., None]
    out = np.log(n) + xm + 0.5 * (y**2).mean(axis=-1)
    if top >= 3:
        out = out + (y**3).mean(axis=-1) / 6.0
    if top not in (2, 3):
        raise ValueError("top must be 2 or 3")
    return out
