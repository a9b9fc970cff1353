"""Pins for the oracle's gradients of truncated-kernel attention (CPU only).

The pages are silent on gradients; the hand-derived formulas are checked against
central finite differences of the forward oracle (the definition, and the
recursion with an incoming state), a closed form at n = 1 (cumulative mean), the
sum rule of a normalised average (sum_j dv_j = sum_i g_i) and planted mistakes.
"""

import numpy as np
import pytest

import oracle


def _loss(q, k, v, g, n, scale, state0=None):
    if state0 is None:
        o, _ = oracle.truncated_attention(q, k, v, n, scale)
    else:
        o, _ = oracle.recurrent(q, k, v, n, scale, state0)
    return float(np.sum(g * o))


def _fd(f, x, h=1e-6):
    out = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        out[idx] = (f(xp) - f(xm)) / (2 * h)
    return out


def _inputs(seed, N=7, d=3, dv=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, d)) * 0.6
    k = rng.standard_normal((N, d)) * 0.6
    v = rng.standard_normal((N, dv))
    g = rng.standard_normal((N, dv))
    return q, k, v, g


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_gradients_match_finite_differences(n):
    q, k, v, g = _inputs(10 + n)
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, g, n, scale)
    np.testing.assert_allclose(dq, _fd(lambda x: _loss(x, k, v, g, n, scale), q), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dk, _fd(lambda x: _loss(q, x, v, g, n, scale), k), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dv, _fd(lambda x: _loss(q, k, x, g, n, scale), v), rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_gradients_with_an_incoming_state(n):
    # the recursion continued from a state (states add across chunks): gradients of q, k, v and of
    # the state itself against finite differences of the forward recursion
    q, k, v, g = _inputs(20 + n, N=6)
    qa, ka, va, _ = _inputs(30 + n, N=5)
    state0 = oracle.state(ka, va, n)
    scale = 0.8
    dq, dk, dv, dst = oracle.attention_backward_from_state(q, k, v, g, n, scale, state0)
    np.testing.assert_allclose(dq, _fd(lambda x: _loss(x, k, v, g, n, scale, state0), q), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dk, _fd(lambda x: _loss(q, x, v, g, n, scale, state0), k), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dv, _fd(lambda x: _loss(q, k, x, g, n, scale, state0), v), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dst, _fd(lambda x: _loss(q, k, v, g, n, scale, x), state0), rtol=1e-6, atol=1e-8)


def test_n1_closed_form():
    # n = 1: o_i is the mean of v_0..v_i, so q and k get no gradient and dv_j = sum_{i>=j} g_i / (i+1)
    q, k, v, g = _inputs(40, N=9)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, 1)
    assert np.all(dq == 0) and np.all(dk == 0)
    want = np.array([sum(g[i] / (i + 1) for i in range(j, 9)) for j in range(9)])
    np.testing.assert_allclose(dv, want, rtol=1e-14, atol=0)


@pytest.mark.parametrize("n", [2, 3, 5])
def test_value_gradients_sum_to_the_upstream_gradient(n):
    # each o_i is an average with weights summing to one, so shifting every v_j by c shifts o_i by c
    q, k, v, g = _inputs(50 + n, N=12, d=4, dv=3)
    dv = oracle.attention_backward(q, k, v, g, n, 0.5)[2]
    np.testing.assert_allclose(dv.sum(0), g.sum(0), rtol=1e-12, atol=1e-12)


def test_planted_mistakes_are_caught():
    # dropping the normaliser's term (delta) or using K_n for K_n' moves dq away from the differences
    q, k, v, g = _inputs(60)
    n, scale = 3, 0.7
    fd = _fd(lambda x: _loss(x, k, v, g, n, scale), q)
    s = scale * (q @ k.T)
    mask = np.tril(np.ones((7, 7), dtype=bool))
    w = np.where(mask, oracle.truncated_kernel(s, n), 0.0)
    den = w.sum(1)
    o = (w @ v) / den[:, None]
    gh = g / den[:, None]
    no_delta = np.where(mask, gh @ v.T, 0.0) * oracle.truncated_kernel(s, n - 1)
    assert np.max(np.abs(scale * (no_delta @ k) - fd)) > 1e-3
    delta = np.sum(g * o, 1) / den
    wrong_deriv = np.where(mask, gh @ v.T - delta[:, None], 0.0) * oracle.truncated_kernel(s, n)
    assert np.max(np.abs(scale * (wrong_deriv @ k) - fd)) > 1e-3


def test_dq_rows_form_matches_full():
    q, k, v, g = _inputs(70, N=20, d=4, dv=3)
    dq = oracle.attention_backward(q, k, v, g, 3, 0.6)[0]
    rows = [0, 5, 19, 11]
    np.testing.assert_allclose(oracle.attention_backward_dq_rows(q, k, v, g, 3, rows, 0.6), dq[rows], rtol=1e-12,
                               atol=1e-14)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("with_state", [False, True])
def test_magnitudes_bound_the_gradients(n, with_state):
    # the magnitudes are sums of absolute values of the gradients' terms, so they dominate the
    # gradients entry by entry (raw scores with a negative scale: every sign shows up)
    q, k, v, g = _inputs(80 + n, N=9, d=3, dv=2)
    state0 = oracle.state(*_inputs(90 + n, N=4, d=3, dv=2)[1:3], n) if with_state else None
    scale = -0.9
    grads = oracle.attention_backward_from_state(q, k, v, g, n, scale, state0)
    mags = oracle.attention_backward_magnitudes(q, k, v, g, n, scale, state0)
    for got, m in zip(grads, mags):
        assert m.shape == got.shape
        assert np.all(np.abs(got) <= m * (1 + 1e-12) + 1e-15)


def test_magnitudes_closed_forms():
    # n = 1 (weights 1, den_i = i + 1): q and k get no terms at all, and dv_j's terms are g_i / (i + 1)
    q, k, v, g = _inputs(95, N=8)
    mq, mk, mv, _ = oracle.attention_backward_magnitudes(q, k, v, g, 1)
    assert np.all(mq == 0) and np.all(mk == 0)
    want = np.array([sum(np.abs(g[i]) / (i + 1) for i in range(j, 8)) for j in range(8)])
    np.testing.assert_allclose(mv, want, rtol=1e-14, atol=0)
    # all-positive inputs at n = 2 and scale 1: dv's terms have one sign, so its magnitude is |dv|
    qp, kp, vp, gp = (np.abs(x) for x in _inputs(96, N=8))
    dv = oracle.attention_backward(qp, kp, vp, gp, 2)[2]
    np.testing.assert_allclose(oracle.attention_backward_magnitudes(qp, kp, vp, gp, 2)[2], dv, rtol=1e-13)


def test_dq_magnitude_rows_form_matches_full():
    q, k, v, g = _inputs(97, N=20, d=4, dv=3)
    mq = oracle.attention_backward_magnitudes(q, k, v, g, 3, -0.6)[0]
    rows = [0, 7, 19]
    np.testing.assert_allclose(oracle.attention_backward_dq_magnitude_rows(q, k, v, g, 3, rows, -0.6), mq[rows],
                               rtol=1e-12, atol=1e-14)
