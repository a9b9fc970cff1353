"""Pins for the oracle's attention routines (CPU only).

The direct O(N^2) definition is checked against: a hand-worked example, closed
forms at n = 1 (cumulative mean) and n = 2 (linear attention via prefix sums),
a pure-Python math.fsum brute force, the positivity of odd-n truncations, the
Lagrange remainder bound towards exact softmax, and the two numerical claims in
the Abstract of "Expanding Attention" (Huang, arXiv:2610.20637): the recursion
reproduces the truncated kernel (2.2e-16 printed) and states add across chunks
(5.7e-14 printed).
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def test_hand_example():
    g = _golden("hand_examples.json")["attention_d1_n3"]
    o, den = oracle.truncated_attention(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), g["n"], g["scale"])
    np.testing.assert_allclose(o, g["o"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(den, g["den"], rtol=1e-15, atol=0)


def test_kernel_polynomial_values():
    # K_n(s) = sum_{m<n} s^m/m!, compared with explicit powers and factorials.
    s = np.linspace(-3, 3, 61)
    for n in range(1, 8):
        ref = np.array([math.fsum(x ** m / math.factorial(m) for m in range(n)) for x in s])
        np.testing.assert_allclose(oracle.truncated_kernel(s, n), ref, rtol=1e-14, atol=1e-15)


def test_n1_is_cumulative_mean():
    # K_1 = 1: every visible key has weight 1, o_i = mean(v_0..v_i) (inclusive causality).
    x = synth.make_qkv(1, 1, 1, 100, 4, 3)
    o, den = oracle.truncated_attention(x.q64[0, 0], x.k64[0, 0], x.v64[0, 0], 1)
    cnt = np.arange(1, 101)[:, None]
    np.testing.assert_allclose(o, np.cumsum(x.v64[0, 0], axis=0) / cnt, rtol=1e-13)
    np.testing.assert_allclose(den, np.arange(1, 101), rtol=0)


@pytest.mark.parametrize("scale", [1.0, 0.25])
def test_n2_is_linear_attention(scale):
    # K_2(s) = 1 + s: linear attention with feature [1, x] evaluated with prefix sums.
    x = synth.make_qkv(1, 1, 1, 300, 4, 5, unit_norm=False)
    q, k, v = x.q64[0, 0], x.k64[0, 0], x.v64[0, 0]
    kv = np.cumsum(k[:, :, None] * v[:, None, :], axis=0)
    ks = np.cumsum(k, axis=0)
    vs = np.cumsum(v, axis=0)
    cnt = np.arange(1, 301)
    num = vs + scale * np.einsum("id,idv->iv", q, kv)
    den = cnt + scale * np.einsum("id,id->i", q, ks)
    o, d = oracle.truncated_attention(q, k, v, 2, scale)
    np.testing.assert_allclose(d, den, rtol=1e-12)
    np.testing.assert_allclose(o, num / den[:, None], rtol=1e-9, atol=1e-12)


def _bruteforce(q, k, v, n, scale):
    """Pure-Python triple loop with math.fsum (no numpy arithmetic)."""
    N, dv = len(q), len(v[0])
    out = []
    for i in range(N):
        ws = []
        for j in range(i + 1):
            s = scale * math.fsum(q[i][t] * k[j][t] for t in range(len(q[i])))
            ws.append(math.fsum(s ** m / math.factorial(m) for m in range(n)))
        den = math.fsum(ws)
        out.append([math.fsum(ws[j] * v[j][c] for j in range(i + 1)) / den for c in range(dv)])
    return np.array(out)


@pytest.mark.parametrize("n", [1, 3, 4])
def test_tiny_config_against_fsum_bruteforce(n):
    # The tiny configuration: N = 256, d_k = d_v = 4, unit-norm q, k.
    x = synth.make_qkv(1, 1, 1, 256, 4, 4)
    q, k, v = x.q64[0, 0], x.k64[0, 0], x.v64[0, 0]
    ref = _bruteforce(q.tolist(), k.tolist(), v.tolist(), n, 1.0)
    o, _ = oracle.truncated_attention(q, k, v, n, 1.0, block=64)
    assert _rel(o, ref) < 1e-14


def test_row_and_decode_forms_match_full():
    x = synth.make_qkv(2, 1, 1, 400, 16, 8)
    q, k, v = x.q64[0, 0], x.k64[0, 0], x.v64[0, 0]
    o, den = oracle.truncated_attention(q, k, v, 3)
    rows = [0, 1, 63, 64, 199, 399]
    o_r, den_r = oracle.truncated_attention_rows(q, k, v, 3, rows)
    np.testing.assert_allclose(o_r, o[rows], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(den_r, den[rows], rtol=1e-13)
    o_t, den_t = oracle.decode_reference(q[250], k[:251], v[:251], 3)
    np.testing.assert_allclose(o_t, o[250], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("n", [1, 3, 5, 7])
def test_odd_n_is_positive_everywhere(n):
    # Truncating at an even highest order (odd n) keeps K_n(s) > 0 for all real s
    # (AI Radio transcript: stop at an even highest order; the kexue "Linear Attention"
    # section: the second-order expansion is non-negative).
    s = np.linspace(-60, 60, 24001)
    assert np.all(oracle.truncated_kernel(s, n) > 0)


@pytest.mark.parametrize("n,root", [(2, -1.0), (4, -1.5960716379833215)])
def test_even_n_has_a_real_root(n, root):
    # Odd highest order: K_n changes sign (n = 2: 1 + s at s = -1; n = 4: the real cubic root).
    assert oracle.truncated_kernel(np.array([root - 1e-3]), n)[0] < 0 < oracle.truncated_kernel(np.array([root + 1e-3]), n)[0]


def _bruteforce_softmax(q, k, v, scale):
    out = []
    for i in range(len(q)):
        s = [scale * math.fsum(a * b for a, b in zip(q[i], k[j])) for j in range(i + 1)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        den = math.fsum(e)
        out.append([math.fsum(e[j] * v[j][c] for j in range(i + 1)) / den for c in range(len(v[0]))])
    return np.array(out)


def test_softmax_against_bruteforce():
    x = synth.make_qkv(3, 1, 1, 64, 4, 3, unit_norm=False)
    q, k, v = x.q64[0, 0], x.k64[0, 0], x.v64[0, 0]
    ref = _bruteforce_softmax(q.tolist(), k.tolist(), v.tolist(), 0.5)
    assert _rel(oracle.softmax_attention(q, k, v, 0.5, block=16), ref) < 1e-13


def test_softmax_rows_form_matches_full():
    x = synth.make_qkv(7, 1, 1, 300, 8, 5, unit_norm=False)
    q, k, v = x.q64[0, 0], x.k64[0, 0], x.v64[0, 0]
    rows = [0, 1, 150, 299, 64]
    full = oracle.softmax_attention(q, k, v, 0.6)
    np.testing.assert_allclose(oracle.softmax_attention_rows(q, k, v, rows, 0.6), full[rows], rtol=1e-13, atol=1e-15)


def test_converges_to_softmax_within_lagrange_bound():
    # Abstract: accuracy improves exponentially in n.  For |s| <= smax the relative kernel
    # error is delta_n <= e^{2 smax} smax^n / n! (Lagrange remainder), and the output error
    # is at most 2 delta/(1-delta) * max_j ||v_j - o_i||.
    x = synth.make_qkv(5, 1, 1, 256, 16, 8)
    q, k, v = x.q64[0, 0], x.k64[0, 0], x.v64[0, 0]
    ref = oracle.softmax_attention(q, k, v)
    smax = float(np.max(np.abs(np.tril(q @ k.T))))
    assert smax <= 1.0 + 1e-12
    spread = max(float(np.max(np.linalg.norm(v[: i + 1] - ref[i], axis=1))) for i in range(256))
    errs = []
    for n in range(1, 11):
        o, _ = oracle.truncated_attention(q, k, v, n)
        err = float(np.max(np.linalg.norm(o - ref, axis=1)))
        delta = math.exp(2 * smax) * smax ** n / math.factorial(n)
        if delta < 1:
            assert err <= 2 * delta / (1 - delta) * spread
        errs.append(err)
    assert errs[-1] < 1e-6
    for a, b in zip(errs[2:], errs[3:]):
        assert b < a


def test_raw_scores_leave_the_accurate_region():
    # Abstract: without q/k normalisation the argument exceeds the convergence radius and
    # adding terms stops helping (qualitative).  Raw N(0,1) q, k with scale 1/sqrt(d_k)
    # give errors far above the normalised case at every 2 <= n <= 5 (at n = 1 both are the
    # plain cumulative mean, whatever the scores).
    unit = synth.make_qkv(5, 1, 1, 256, 16, 8)
    raw = synth.make_qkv(5, 1, 1, 256, 16, 8, unit_norm=False)
    for n in range(2, 6):
        ou, _ = oracle.truncated_attention(unit.q64[0, 0], unit.k64[0, 0], unit.v64[0, 0], n)
        eu = _rel(ou, oracle.softmax_attention(unit.q64[0, 0], unit.k64[0, 0], unit.v64[0, 0]))
        o_r, _ = oracle.truncated_attention(raw.q64[0, 0], raw.k64[0, 0], raw.v64[0, 0], n, 0.25)
        er = _rel(o_r, oracle.softmax_attention(raw.q64[0, 0], raw.k64[0, 0], raw.v64[0, 0], 0.25))
        assert er > 10 * eu


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_recursion_equals_truncated_kernel(n):
    # Abstract: the recursion is lossless with respect to the truncated kernel (2.2e-16, float64).
    bar = 1e-14
    assert _golden("pages_figures.json")["recursion_vs_truncated_kernel_float64"]["value"] < bar
    x = synth.make_qkv(2, 1, 1, 512, 16, 16)
    q, k, v = x.q64[0, 0], x.k64[0, 0], x.v64[0, 0]
    o_rec, S = oracle.recurrent(q, k, v, n)
    o_dir, _ = oracle.truncated_attention(q, k, v, n)
    assert _rel(o_rec, o_dir) < bar
    assert S.shape == (oracle.feature_width(n, 16), 17)


def test_state_hand_example():
    # Two tokens worked by hand: the state is the sum of phi(k_j) [v_j, 1]^T, z in the last column.
    g = _golden("hand_examples.json")["state_d2_n3_two_tokens"]
    k, v, want = np.array(g["k"]), np.array(g["v"]), np.array(g["state"])
    np.testing.assert_allclose(oracle.state(k, v, g["n"]), want, rtol=1e-15, atol=1e-15)
    # the rank-one recursion reaches the same state token by token
    _, S = oracle.recurrent(np.zeros_like(k), k, v, g["n"])
    np.testing.assert_allclose(S, want, rtol=1e-15, atol=1e-15)
    # planted mistakes the fixture catches: the last token left out; features without 1/sqrt(alpha!)
    assert not np.allclose(oracle.state(k[:1], v[:1], 3), want)
    bare = np.array([[1.0, x0, x1, x0 * x0, x0 * x1, x1 * x1] for x0, x1 in k])
    assert not np.allclose(bare.T @ np.concatenate([v, np.ones((2, 1))], axis=1), want)


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_state_equals_the_recursions_final_state(n):
    # The closed-form sum (one matrix product over all tokens) against the token-by-token rank-one
    # updates of the recursion: two separate statements of the same state (Abstract: the recurrent
    # states are sums over the causal history).
    x = synth.make_qkv(6, 1, 1, 700, 16, 8)
    k, v = x.k64[0, 0], x.v64[0, 0]
    _, S = oracle.recurrent(x.q64[0, 0], k, v, n)
    assert _rel(oracle.state(k, v, n), S) < 1e-14
    # the normaliser column counts tokens in its constant-feature entry
    assert S[0, -1] == 700


@pytest.mark.parametrize("chunk", [1, 37, 64, 128, 1000])
def test_states_add_across_chunks(chunk):
    # Abstract: states are additive across chunks (5.7e-14), so prefill admits a parallel scan.
    bar = 1e-13
    assert _golden("pages_figures.json")["chunk_additivity_float64"]["value"] < bar
    x = synth.make_qkv(2, 1, 1, 1000, 16, 8)
    k, v = x.k64[0, 0], x.v64[0, 0]
    full = oracle.state(k, v, 3)
    assert _rel(oracle.chunked_state(k, v, 3, chunk), full) < bar
    # The last column is the normaliser z = sum_j phi(k_j); its first entry counts tokens.
    assert full[0, -1] == 1000


def test_recursion_resumes_from_a_state():
    # The state is the whole memory of the prefix: run(N1) then run(N2 | state) = run(N1+N2).
    x = synth.make_qkv(2, 1, 1, 300, 16, 8)
    q, k, v = x.q64[0, 0], x.k64[0, 0], x.v64[0, 0]
    o_all, S_all = oracle.recurrent(q, k, v, 3)
    o1, S1 = oracle.recurrent(q[:120], k[:120], v[:120], 3)
    o2, S2 = oracle.recurrent(q[120:], k[120:], v[120:], 3, state0=S1)
    assert _rel(np.vstack([o1, o2]), o_all) < 1e-14
    assert _rel(S2, S_all) < 1e-14


def test_planted_mistakes_are_caught():
    # Each plausible slip in the definition must move the hand example: a dropped term,
    # exclusive causality, a missing normaliser.
    g = _golden("hand_examples.json")["attention_d1_n3"]
    q, k, v = (np.array(g[c]) for c in "qkv")
    good, _ = oracle.truncated_attention(q, k, v, 3)
    dropped, _ = oracle.truncated_attention(q, k, v, 2)
    assert np.max(np.abs(dropped - np.array(g["o"]))) > 1e-3
    s = q @ k.T
    w = oracle.truncated_kernel(s, 3)
    excl = np.tril(w, -1)
    with np.errstate(invalid="ignore", divide="ignore"):
        o_excl = (excl @ v) / excl.sum(1, keepdims=True)
    assert not np.allclose(o_excl[1:], good[1:])
    assert not np.allclose(np.tril(w) @ v, good)
