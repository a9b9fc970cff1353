"""Pins for the oracle's monomial tables and feature map (CPU only).

Each check compares the oracle with something other than itself: the width
formula and state size printed in the Abstract of "Expanding Attention"
(Huang, arXiv:2610.20637), a second table generator written differently,
hand-worked fixtures, closed forms of the tensor-power inner product, explicit
Kronecker tensor powers, and the SVD rank claim of the Abstract.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _exponent_vectors(d, m):
    """All alpha in N^d with |alpha| = m, by recursion on the first coordinate (independent generator)."""
    if d == 1:
        return [(m,)]
    out = []
    for a0 in range(m + 1):
        for rest in _exponent_vectors(d - 1, m - a0):
            out.append((a0,) + rest)
    return out


def _tuple_of(alpha):
    return tuple(i for i, a in enumerate(alpha) for _ in range(a))


@pytest.mark.parametrize("d", [1, 2, 4, 16])
@pytest.mark.parametrize("m", [0, 1, 2, 3, 4])
def test_width_formula(d, m):
    # Abstract: the m-th state is binom(d+m-1, m) wide.
    assert len(oracle.monomials(d, m)) == math.comb(d + m - 1, m)


def test_state_size_printed_in_abstract():
    g = _golden("pages_figures.json")["state_elems_per_head"]
    W = oracle.feature_width(g["n"], g["d_k"])
    assert W * (g["d_v"] + 1) == g["value"] == 9945
    assert [len(oracle.monomials(16, m)) for m in range(5)] == [1, 16, 136, 816, 3876]
    assert [oracle.feature_width(n, 16) for n in range(1, 6)] == [1, 17, 153, 969, 4845]
    assert oracle.feature_width(3, 4) == 15


@pytest.mark.parametrize("d,n", [(1, 5), (3, 4), (4, 5), (16, 4)])
def test_table_order_against_independent_generator(d, n):
    expected = []
    for m in range(n):
        tuples = sorted(_tuple_of(a) for a in _exponent_vectors(d, m))
        expected.extend(tuples)
    got = [tup for (_, tup, _) in oracle.feature_table(n, d)]
    assert got == expected
    # within each order: strictly increasing (lexicographic, no duplicates), non-decreasing tuples
    for m in range(n):
        block = [t for t in got if len(t) == m]
        assert all(a < b for a, b in zip(block, block[1:]))
        assert all(list(t) == sorted(t) for t in block)


def test_tables_hand_fixture():
    g = _golden("hand_examples.json")["tables_d3_n4"]
    tab = oracle.feature_table(g["n"], g["d"])
    assert [list(t) for (_, t, _) in tab] == g["tuples"]
    for (_, _, c), af in zip(tab, g["alpha_factorial"]):
        assert c == 1.0 / math.sqrt(float(af))
    idx = oracle.index_table(g["n"], g["d"])
    assert idx.dtype == np.int32 and idx.shape == (20, 3)
    for row, t in zip(idx, g["tuples"]):
        assert list(row[: len(t)]) == t and all(row[len(t):] == -1)


def test_features_hand_fixture():
    g = _golden("hand_examples.json")["features_d2_n3"]
    px = oracle.features(np.array(g["x"]), g["n"])
    py = oracle.features(np.array(g["y"]), g["n"])
    np.testing.assert_allclose(px, g["phi_x"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(py, g["phi_y"], rtol=1e-15, atol=0)
    assert abs(px @ py - g["inner"]) < 1e-14


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_feature_inner_product_is_truncated_exponential(n):
    # <phi(q), phi(k)> = sum_{m<n} (q.k)^m / m!  (the factorisation in the Abstract)
    rng = np.random.default_rng(11)
    q = rng.standard_normal((40, 16)) * 0.3
    k = rng.standard_normal((40, 16)) * 0.3
    lhs = np.einsum("iw,iw->i", oracle.features(q, n), oracle.features(k, n))
    for i in range(40):
        s = float(q[i] @ k[i])
        rhs = math.fsum(s ** m / math.factorial(m) for m in range(n))
        assert abs(lhs[i] - rhs) <= 1e-14 * max(1.0, abs(rhs))


@pytest.mark.parametrize("m", [0, 1, 2, 3, 4])
def test_feature_norm_closed_form(m):
    # ||phi_m(x)||^2 = ||x||^(2m) / m!   (<phi_m(x), phi_m(x)> = (x.x)^m/m!)
    rng = np.random.default_rng(12 + m)
    x = rng.standard_normal((25, 16))
    fm = oracle.features_by_order(x, m + 1)[m]
    lhs = (fm * fm).sum(axis=1)
    rhs = (x * x).sum(axis=1) ** m / math.factorial(m)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-13)


def _kron_power(x, m):
    out = np.ones(1)
    for _ in range(m):
        out = np.kron(out, x)
    return out


@pytest.mark.parametrize("d,m", [(2, 2), (3, 2), (3, 3), (4, 3), (2, 4)])
def test_features_equal_kronecker_tensor_powers(d, m):
    # <phi_m(q), phi_m(k)> = <q^{(x)m}, k^{(x)m}> / m!  with explicit d^m-entry tensor powers
    rng = np.random.default_rng(100 + 10 * d + m)
    for _ in range(5):
        q = rng.standard_normal(d)
        k = rng.standard_normal(d)
        lhs = oracle.features_by_order(q, m + 1)[m] @ oracle.features_by_order(k, m + 1)[m]
        rhs = _kron_power(q, m) @ _kron_power(k, m) / math.factorial(m)
        assert abs(lhs - rhs) <= 1e-13 * max(1.0, abs(rhs))


@pytest.mark.parametrize("d,m", [(4, 1), (4, 2), (4, 3), (3, 4)])
def test_svd_rank_equals_width(d, m):
    # Abstract: the binom(d+m-1, m) width bound is confirmed by SVD.  The N x d^m matrix of
    # tensor powers k_j^{(x)m} has that rank, and the oracle's phi_m spans exactly its row space.
    rng = np.random.default_rng(7 + d + m)
    N = 200
    k = rng.standard_normal((N, d))
    kron = np.stack([_kron_power(k[j], m) for j in range(N)])
    phi = oracle.features_by_order(k, m + 1)[m]
    width = math.comb(d + m - 1, m)

    def rank(a):
        s = np.linalg.svd(a, compute_uv=False)
        return int((s > s[0] * 1e-10).sum())

    assert phi.shape[1] == width
    assert rank(kron) == width
    assert rank(phi) == width
    assert rank(np.hstack([kron, phi])) == width
