"""Monomial index tables of the symmetric tensor-power features (oracle; test infrastructure only).

Source: "Expanding Attention: A Taylor-Series Route to Linear-Time Transformers
with a Fixed Number of Recurrent States" (Huang, arXiv:2610.20637), Abstract:
each Taylor term (q.k)^m is factorised as an inner product of m-th tensor
powers, and the m-th state is binom(d+m-1, m) wide.  The width is the number of
distinct entries of the symmetric tensor x^{(x)m}: one per multiset
{i_1 <= ... <= i_m} of coordinates, i.e. one per exponent vector alpha with
|alpha| = m.  The scholarbro listing of the same abstract prints the formula
cleanly.

Readings taken where the pages are silent:

* Order: orders m = 0 .. n-1 ascending ("n terms" includes the constant term);
  within an order, non-decreasing coordinate tuples in lexicographic order
  (the order of ``itertools.combinations_with_replacement``).
* Coefficient: the entry for multiset alpha appears m!/alpha! times in
  x^{(x)m}; folding that multiplicity and the 1/m! of the Taylor term into the
  two factors symmetrically gives c_alpha = sqrt(m!/alpha! / m!) = 1/sqrt(alpha!).
  It is evaluated in float64 as ``1.0 / math.sqrt(float(prod(alpha_i!)))``
  (both IEEE-correctly-rounded steps).
"""

import itertools
import math

import numpy as np


def monomials(d, m):
    """Non-decreasing coordinate tuples (i_1 <= ... <= i_m) over range(d), lexicographic.

    There are binom(d+m-1, m) of them (the width formula of the Abstract).
    """
    return list(itertools.combinations_with_replacement(range(d), m))


def exponents(tup, d):
    """Exponent vector alpha (length d) of the monomial named by a coordinate tuple."""
    alpha = [0] * d
    for i in tup:
        alpha[i] += 1
    return alpha


def coefficient(tup, d):
    """c_alpha = 1/sqrt(alpha!) with alpha! = prod_i alpha_i! (float64)."""
    denom = 1
    for a in exponents(tup, d):
        denom *= math.factorial(a)
    return 1.0 / math.sqrt(float(denom))


def feature_table(n, d):
    """[(order m, coordinate tuple, coefficient)] for m = 0..n-1, in feature order."""
    if n < 1 or d < 1:
        raise ValueError("need n >= 1 and d >= 1")
    out = []
    for m in range(n):
        for tup in monomials(d, m):
            out.append((m, tup, coefficient(tup, d)))
    return out


def feature_width(n, d):
    """W = sum_{m<n} binom(d+m-1, m), counted from the table itself."""
    return len(feature_table(n, d))


def index_table(n, d):
    """int32 [W, max(n-1, 1)]: the coordinates of each feature, padded with -1."""
    tab = feature_table(n, d)
    width = max(n - 1, 1)
    out = np.full((len(tab), width), -1, dtype=np.int32)
    for r, (_, tup, _) in enumerate(tab):
        out[r, : len(tup)] = tup
    return out


def coef_table(n, d):
    """float64 [W]: the coefficient of each feature."""
    return np.array([c for (_, _, c) in feature_table(n, d)], dtype=np.float64)
