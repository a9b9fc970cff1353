"""Pins for the oracle's softmax-expanded-about-the-mean attention (CPU only).

Source: Su Jianlin, kexue.fm translation 11814, sections "Basic Expansion",
"Calculating the Gradient" and "Linear Attention".  The direct definition is
checked against: hand-worked fractions, the page's two claims about the
truncated expansion (it is the gradient of the truncated logsumexp series, and
its weights still sum to one), its convergence order towards exact softmax, the
degenerate cases (one key, equal keys), a closed form through prefix moment sums
(the page's "linear attention" reading) and planted mistakes.
"""

import json
import os

import numpy as np
import pytest

from oracle import centered

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "centered_examples.json")) as f:
        return json.load(f)


def test_hand_weights():
    g = _golden()["weights_x012"]
    for order in (1, 2):
        want = np.array([p / q for p, q in g[f"order{order}"]])
        np.testing.assert_allclose(centered.centered_weights(np.array(g["x"]), order), want, rtol=0, atol=1e-15)


def test_hand_attention():
    g = _golden()["attention_d1"]
    q, k, v = (np.array(g[c]) for c in "qkv")
    for order in (1, 2):
        want = np.array([[p / r for p, r in row] for row in g[f"order{order}"]])
        got = centered.centered_attention(q, k, v, order, g["scale"])
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("order", [1, 2])
def test_weights_sum_to_one(order):
    # "Calculating the Gradient": every truncation keeps the components summing to one.
    rng = np.random.default_rng(1)
    for n in (1, 2, 3, 17, 200):
        x = rng.standard_normal((5, n)) * 2.0
        np.testing.assert_allclose(centered.centered_weights(x, order).sum(-1), 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("order", [1, 2])
def test_weights_are_the_gradient_of_the_lse_series(order):
    # "Calculating the Gradient": softmax = grad logsumexp, so the softmax expansion through y^order is
    # the gradient of the logsumexp series through y^(order+1).  Central differences (h = 1e-5) on
    # the separately written series.
    rng = np.random.default_rng(2)
    h = 1e-5
    for n in (2, 5, 33):
        x = rng.standard_normal(n)
        grad = np.empty(n)
        for j in range(n):
            e = np.zeros(n)
            e[j] = h
            grad[j] = (centered.lse_series(x + e, order + 1) - centered.lse_series(x - e, order + 1)) / (2 * h)
        np.testing.assert_allclose(centered.centered_weights(x, order), grad, rtol=0, atol=1e-8)


@pytest.mark.parametrize("order", [1, 2])
def test_converges_to_softmax_at_its_order(order):
    # Truncating after y^order leaves an error of order eps^(order+1) when the scores shrink by eps.
    rng = np.random.default_rng(3)
    x0 = rng.standard_normal(40)

    def err(eps):
        x = eps * x0
        sm = np.exp(x - x.max())
        sm /= sm.sum()
        return np.max(np.abs(centered.centered_weights(x, order) - sm))

    ratios = [err(e) / err(e / 2) for e in (0.04, 0.02, 0.01)]
    for r in ratios:
        assert abs(r - 2.0 ** (order + 1)) < 0.15 * 2.0 ** (order + 1), ratios


def test_lse_series_against_exact_logsumexp():
    # The series itself: its error shrinks as eps^3 (top = 2) and eps^4 (top = 3).
    rng = np.random.default_rng(4)
    x0 = rng.standard_normal(30)
    for top in (2, 3):
        e1 = abs(centered.lse_series(0.02 * x0, top) - np.log(np.exp(0.02 * x0).sum()))
        e2 = abs(centered.lse_series(0.01 * x0, top) - np.log(np.exp(0.01 * x0).sum()))
        assert abs(e1 / e2 - 2.0 ** (top + 1)) < 0.15 * 2.0 ** (top + 1)


@pytest.mark.parametrize("order", [1, 2])
def test_degenerate_cases(order):
    rng = np.random.default_rng(5)
    q = rng.standard_normal((20, 4))
    v = rng.standard_normal((20, 3))
    # one key: o_0 = v_0
    k = rng.standard_normal((20, 4))
    o = centered.centered_attention(q, k, v, order)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    # equal keys: every score equals the mean, so the weights are uniform: o_i = mean(v_0..v_i)
    ke = np.tile(k[:1], (20, 1))
    o = centered.centered_attention(q, ke, v, order)
    np.testing.assert_allclose(o, np.cumsum(v, 0) / np.arange(1, 21)[:, None], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("order", [1, 2])
def test_linear_attention_closed_form(order):
    # "Linear Attention": with prefix sums c = i+1, s1 = sum k_j, M = sum k_j k_j^T, V0 = sum v_j,
    # V1 = sum k_j v_j^T and V2 = sum (a.k_j)^2 v_j (an inner product of outer products, a = sigma q_i):
    #   u = a.s1 / c,  d2 = a^T M a / 2,  P1 = a^T V1,  P2 = V2 / 2
    #   order 1: o = ((1 - u) V0 + P1) / c
    #   order 2: o = ((1 - u + u^2 - d2/c) V0 + (1 - u) P1 + P2) / c
    rng = np.random.default_rng(6)
    N, d, dv, sigma = 50, 5, 3, 0.7
    q, k, v = rng.standard_normal((N, d)), rng.standard_normal((N, d)), rng.standard_normal((N, dv))
    want = centered.centered_attention(q, k, v, order, sigma)
    for i in range(N):
        a = sigma * q[i]
        kk, vv = k[: i + 1], v[: i + 1]
        c = i + 1
        s1, M = kk.sum(0), kk.T @ kk
        V0, V1 = vv.sum(0), kk.T @ vv
        outer = np.einsum("j,jab->jab", np.ones(c), np.einsum("ja,jb->jab", kk, kk))
        V2 = np.einsum("ab,jab,jc->c", np.outer(a, a), outer, vv)
        u, d2, P1, P2 = a @ s1 / c, a @ M @ a / 2, a @ V1, V2 / 2
        if order == 1:
            o = ((1 - u) * V0 + P1) / c
        else:
            o = ((1 - u + u * u - d2 / c) * V0 + (1 - u) * P1 + P2) / c
        np.testing.assert_allclose(o, want[i], rtol=1e-11, atol=1e-12)


def test_rows_form_matches_full():
    rng = np.random.default_rng(7)
    q, k, v = rng.standard_normal((30, 4)), rng.standard_normal((30, 4)), rng.standard_normal((30, 2))
    full = centered.centered_attention(q, k, v, 2, 0.5)
    rows = [0, 7, 29, 13]
    np.testing.assert_allclose(centered.centered_attention_rows(q, k, v, 2, rows, 0.5), full[rows], rtol=0, atol=0)


def test_planted_mistakes_are_caught():
    # A dropped mean(y^2), a sum in place of a mean, and centring on the wrong quantity each break a pin.
    x = np.array([0.0, 1.0, 2.0])
    y = x - x.mean()
    no_mean = (1 + y + 0.5 * y * y) / 3
    assert abs(no_mean.sum() - 1) > 1e-3
    summed = (1 + y + 0.5 * (y * y - (y * y).sum())) / 3
    assert abs(summed.sum() - 1) > 1e-3
    g = _golden()["weights_x012"]
    want = np.array([p / q for p, q in g["order2"]])
    uncentred = (1 + x + 0.5 * (x * x - (x * x).mean())) / 3
    assert np.max(np.abs(uncentred - want)) > 1e-3


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("scale", [1.0, -0.7])
def test_magnitudes_bound_the_output(order, scale):
    # sums of absolute values of the output's terms dominate the output entry by entry
    rng = np.random.default_rng(30 + order)
    q, k, v = rng.standard_normal((40, 5)), rng.standard_normal((40, 5)), rng.standard_normal((40, 3))
    o = centered.centered_attention(q, k, v, order, scale)
    m = centered.centered_magnitudes(q, k, v, order, scale)
    assert m.shape == o.shape
    assert np.all(np.abs(o) <= m * (1 + 1e-12))


def test_magnitudes_single_key_closed_form():
    # one key: c = 1 and u_bar = s_bar.  Order 1: g0 = 1 + s_bar, g1 = 1.  Order 2: g0 = 1 + s_bar +
    # s_bar^2 + s_bar^2 / 2, g1 = 1 + s_bar, g2 = 1.  The magnitude is (g0 + g1 s_bar + g2 s_bar^2 / 2) |v_0|.
    q, k, v = np.array([[0.5, -2.0]]), np.array([[1.0, 1.5]]), np.array([[2.0, -3.0]])
    sb = 0.5 * 1.0 + 2.0 * 1.5
    av = np.abs(v[0])
    np.testing.assert_allclose(centered.centered_magnitudes(q, k, v, 1)[0], (1 + sb) * av + sb * av, rtol=1e-15)
    g0 = 1 + sb + sb * sb + 0.5 * sb * sb
    want2 = g0 * av + (1 + sb) * sb * av + 0.5 * sb * sb * av
    np.testing.assert_allclose(centered.centered_magnitudes(q, k, v, 2)[0], want2, rtol=1e-15)
