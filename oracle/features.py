"""Symmetric tensor-power feature map phi (oracle; test infrastructure only).

Source: "Expanding Attention: A Taylor-Series Route to Linear-Time Transformers
with a Fixed Number of Recurrent States" (Huang, arXiv:2610.20637), Abstract:
each Taylor term s^m/m! of the kernel is an inner product of tensor powers,
reduced by symmetry to binom(d+m-1, m) monomials.  Here

    phi_m(x)_alpha = c_alpha * prod_i x_i^{alpha_i},   c_alpha = 1/sqrt(alpha!)

so that <phi_m(q), phi_m(k)> = (q.k)^m / m! and phi = [phi_0, ..., phi_{n-1}].
The feature order and coefficients are those of ``oracle.tables``.
"""

import numpy as np

from .tables import feature_table


def features_by_order(x, n):
    """List [phi_0(x), ..., phi_{n-1}(x)], each [..., binom(d+m-1, m)] float64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    tab = feature_table(n, d)
    per_order = [[] for _ in range(n)]
    for m, tup, c in tab:
        col = np.full(x.shape[:-1], c, dtype=np.float64)
        for i in tup:
            col = col * x[..., i]
        per_order[m].append(col)
    return [np.stack(cols, axis=-1) for cols in per_order]


def features(x, n):
    """phi(x) = concat_m phi_m(x): [..., W] float64, W = sum_{m<n} binom(d+m-1, m)."""
    return np.concatenate(features_by_order(x, n), axis=-1)
