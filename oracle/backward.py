"""Gradients of truncated-kernel causal attention (oracle; test infrastructure only).

Source: "Expanding Attention" (Huang, arXiv:2610.20637), Abstract, for the forward
definition (see ``oracle.attention``); the pages are silent on gradients, so this
module differentiates that definition by hand, and the tests pin it against
central finite differences of the forward oracle.

For one head, with w_ij = K_n(s_ij), s_ij = sigma q_i . k_j (j <= i),
den_i = sum_j w_ij, o_i = sum_j w_ij v_j / den_i and an upstream gradient g_i:

    dw_ij = g_i . (v_j - o_i) / den_i          (j <= i)
    dv_j  = sum_{i>=j} w_ij g_i / den_i
    ds_ij = dw_ij K_{n-1}(s_ij)                  (K_n' = K_{n-1}; K_0 = 0)
    dq_i  = sigma sum_{j<=i} ds_ij k_j
    dk_j  = sigma sum_{i>=j} ds_ij q_i

``attention_backward`` writes these out directly in O(N^2).  With a state S0, z0
carried in from earlier tokens (the forward's ``recurrent`` with ``state0``), the
extra history adds phi(sigma q_i) . [S0 | z0] to the numerator and denominator of
every row; ``attention_backward_from_state`` covers that case and also returns the
gradient with respect to [S0 | z0]:

    dS0 = sum_i phi(sigma q_i) g_i^T / den_i,   dz0 = - sum_i phi(sigma q_i) (g_i . o_i) / den_i
"""

import numpy as np

from .attention import truncated_kernel
from .features import features
from .tables import feature_table


def _kernel_derivative(s, n):
    """K_n'(s) = K_{n-1}(s) (zero for n = 1)."""
    if n == 1:
        return np.zeros_like(np.asarray(s, dtype=np.float64))
    return truncated_kernel(s, n - 1)


def attention_backward(q, k, v, g, n, scale=1.0):
    """(dq, dk, dv) of L = sum_i g_i . o_i for one head, from an empty history; float64."""
    return attention_backward_from_state(q, k, v, g, n, scale)[:3]


def attention_backward_from_state(q, k, v, g, n, scale=1.0, state0=None):
    """(dq, dk, dv, dstate0) with an incoming state [W, d_v + 1] (zero if None); float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    N, dv_ = v.shape
    s = scale * (q @ k.T)
    mask = np.tril(np.ones((N, N), dtype=bool))
    w = np.where(mask, truncated_kernel(s, n), 0.0)
    num = w @ v
    den = w.sum(axis=1)
    fq = features(scale * q, n)
    if state0 is not None:
        st = np.asarray(state0, dtype=np.float64)
        num = num + fq @ st[:, :dv_]
        den = den + fq @ st[:, dv_]
    o = num / den[:, None]
    gh = g / den[:, None]                      # dL/dnum_i
    delta = np.sum(g * o, axis=1) / den        # -dL/dden_i
    dw = np.where(mask, gh @ v.T - delta[:, None], 0.0)
    dv = w.T @ gh
    ds = dw * _kernel_derivative(s, n)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    if state0 is not None:
        # the state enters through phi(sigma q_i): d/dq_i of phi(a_i) . (S0 gh_i - z0 delta_i), a = sigma q
        y = st[:, :dv_] @ gh.T - np.outer(st[:, dv_], delta)  # [W, N]
        dq = dq + scale * _feature_vjp(scale * q, y.T, n)
    dstate = np.concatenate([fq.T @ gh, -(fq.T @ delta)[:, None]], axis=1)
    return dq, dk, dv, dstate


def attention_backward_magnitudes(q, k, v, g, n, scale=1.0, state0=None):
    """Per-element magnitudes (mq, mk, mv, mstate) of the sums behind (dq, dk, dv, dstate0); float64.

    The same sums as ``attention_backward_from_state`` with every factor replaced by its absolute
    value: scores by s_bar_ij = |sigma| |q_i| . |k_j| (componentwise absolute values), the weights
    K_n(s) and K_{n-1}(s) by K_n(s_bar) and K_{n-1}(s_bar), and g_i . (v_j - o_i) by
    |g_i| . |v_j| + |g_i| . o_bar_i with o_bar_i = sum_j K_n(s_bar_ij) |v_j| / den_i (plus the
    incoming state's part, |phi(sigma q_i)| |S0|).  Since |s^m| <= s_bar^m term by term and
    phi(|x|) = |phi(x)| (the coefficients are positive), sum_f |phi_f(a)| |phi_f(k)| = K_n(s_bar):
    each entry is at least the sum of the absolute values of the terms that the direct form, or the
    factorised state form, adds up to that entry.  A float32 evaluation in any summation order is
    therefore off by at most a multiple of the float32 unit roundoff times these (the multiple grows
    with the depth of the summation and the number of roundings per term, not with cancellation).
    den_i is the true (signed) normaliser.  Not a result to reproduce: the bound parity tests scale
    their per-row bars by where a row's gradient is a small difference of large terms."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    N, dv_ = v.shape
    sig = abs(scale)
    mask = np.tril(np.ones((N, N), dtype=bool))
    s = scale * (q @ k.T)
    w = np.where(mask, truncated_kernel(s, n), 0.0)
    den = w.sum(axis=1)
    sbar = sig * (np.abs(q) @ np.abs(k).T)
    wbar = np.where(mask, truncated_kernel(sbar, n), 0.0)
    dbar = np.where(mask, np.abs(_kernel_derivative(sbar, n)), 0.0)
    fa = features(sig * np.abs(q), n)  # |phi(sigma q)|
    onum = wbar @ np.abs(v)
    if state0 is not None:
        st = np.abs(np.asarray(state0, dtype=np.float64))
        den = den + features(scale * q, n) @ np.asarray(state0, dtype=np.float64)[:, dv_]
        onum = onum + fa @ st[:, :dv_]
    ad = np.abs(den)
    obar = onum / ad[:, None]
    ghbar = np.abs(g) / ad[:, None]
    dlbar = np.sum(np.abs(g) * obar, axis=1) / ad
    dwbar = np.where(mask, ghbar @ np.abs(v).T + dlbar[:, None], 0.0)
    dsbar = dwbar * dbar
    mq = sig * (dsbar @ np.abs(k))
    mk = sig * (dsbar.T @ np.abs(q))
    mv = wbar.T @ ghbar
    if state0 is not None:
        y = st[:, :dv_] @ ghbar.T + np.outer(st[:, dv_], dlbar)
        mq = mq + sig * _feature_vjp(sig * np.abs(q), y.T, n)
    mstate = np.concatenate([fa.T @ ghbar, (fa.T @ dlbar)[:, None]], axis=1)
    return mq, mk, mv, mstate


def attention_backward_dq_rows(q, k, v, g, n, rows, scale=1.0):
    """dq at the query rows ``rows`` only (empty history): O(N) per row, for sampled checks at sizes
    where the full O(N^2) pass is too large.  g is [N, d_v]; only its rows in ``rows`` matter."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    out = np.empty((len(rows), q.shape[1]))
    for r, i in enumerate(np.asarray(rows, dtype=np.int64)):
        s = scale * (k[: i + 1] @ q[i])
        w = truncated_kernel(s, n)
        den = w.sum()
        o = (w @ v[: i + 1]) / den
        dw = (v[: i + 1] @ g[i] - g[i] @ o) / den
        out[r] = scale * ((dw * _kernel_derivative(s, n)) @ k[: i + 1])
    return out


def attention_backward_dq_magnitude_rows(q, k, v, g, n, rows, scale=1.0):
    """The dq magnitudes of ``attention_backward_magnitudes`` at the query rows ``rows`` only (empty
    history), O(N) per row, for sampled checks at large N."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    sig = abs(scale)
    out = np.empty((len(rows), q.shape[1]))
    for r, i in enumerate(np.asarray(rows, dtype=np.int64)):
        den = truncated_kernel(scale * (k[: i + 1] @ q[i]), n).sum()
        sbar = sig * (np.abs(k[: i + 1]) @ np.abs(q[i]))
        obar = (truncated_kernel(sbar, n) @ np.abs(v[: i + 1])) / abs(den)
        dwbar = (np.abs(v[: i + 1]) @ np.abs(g[i]) + np.abs(g[i]) @ obar) / abs(den)
        out[r] = sig * ((dwbar * np.abs(_kernel_derivative(sbar, n))) @ np.abs(k[: i + 1]))
    return out


def _feature_vjp(x, y, n):
    """sum_f y_f d phi_f(x) / dx, row by row: d/dx_d of c prod_{t in tup} x_t is c times the number of
    times d occurs in tup times the product over tup with one occurrence of d removed."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros_like(x)
    for f, (m, tup, c) in enumerate(feature_table(n, x.shape[1])):
        for d in set(tup):
            rest = list(tup)
            rest.remove(d)
            term = np.full(x.shape[0], c * tup.count(d))
            for t in rest:
                term = term * x[:, t]
            out[:, d] += y[:, f] * term
    return out
