"""Float64 CPU oracle for Taylor-truncated causal attention with recurrent states.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow statement of what the
library computes, used to check it. Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it; the
library and its Python binding never do, and nothing here is shared with the
HIP code (no tables, constants or helpers cross over).

Sources (cited by page title and section; the pages hold prose and formulas,
no code):

* "Expanding Attention: A Taylor-Series Route to Linear-Time Transformers with
  a Fixed Number of Recurrent States" (Z. Huang, arXiv:2610.20637), Abstract --
  the method: the exponential attention kernel is replaced by its Taylor
  polynomial of n terms; each term is written as an inner product of tensor
  powers; the causal history becomes n recurrent states with one rank-one update
  per token; states add across chunks; the m-th state is binom(d+m-1, m) wide.
* The same paper's listing on scholarbro (Abstract, clean LaTeX of the width
  formula) and the "AI Radio" episode page on it (transcript: unit-ratio
  normalisation of q and k, truncation at an even highest order).
* Su Jianlin, kexue.fm translation 11814, section "Linear Attention" -- a
  second-order expansion of exp is non-negative (the "Based" remark); sections
  "Basic Expansion", "Calculating the Gradient" and "Linear Attention" -- the
  softmax expanded about the mean score, a second linear-attention readout of
  the same moment states.

Modules:

* ``tables``    -- monomial index tables and coefficients 1/sqrt(alpha!).
* ``features``  -- the symmetric tensor-power feature map phi.
* ``attention`` -- direct O(N^2) truncated-kernel attention (the definition),
  causal softmax attention, and the separate state / recurrence / chunk routines
  used only to pin the pages' claims.
* ``centered`` -- direct O(N^2) causal attention with the softmax expanded about
  the mean score (orders 1, 2), and the logsumexp series it is the gradient of.
* ``backward`` -- gradients of the truncated-kernel attention (dq, dk, dv, and the
  incoming state's), differentiated by hand from the definition.

Every function that has no independent pin says "parity unpinned" in its
docstring; at present every function is pinned (see tests/test_oracle_*.py).
"""

from .tables import monomials, exponents, coefficient, feature_table, index_table, coef_table, feature_width
from .features import features, features_by_order
from . import centered
from .backward import (attention_backward, attention_backward_from_state, attention_backward_dq_rows,
                       attention_backward_magnitudes, attention_backward_dq_magnitude_rows)
from .centered import centered_weights, centered_attention, centered_attention_rows, centered_magnitudes, lse_series
from .attention import (
    truncated_kernel,
    truncated_attention,
    truncated_attention_rows,
    softmax_attention,
    softmax_attention_rows,
    state,
    recurrent,
    chunked_state,
    decode_reference,
    batched,
)

__all__ = [
    "monomials", "exponents", "coefficient", "feature_table", "index_table", "coef_table", "feature_width",
    "features", "features_by_order",
    "truncated_kernel", "truncated_attention", "truncated_attention_rows", "softmax_attention",
    "softmax_attention_rows",
    "state", "recurrent", "chunked_state", "decode_reference", "batched",
    "centered", "centered_weights", "centered_attention", "centered_attention_rows", "centered_magnitudes",
    "lse_series",
    "attention_backward", "attention_backward_from_state", "attention_backward_dq_rows",
    "attention_backward_magnitudes", "attention_backward_dq_magnitude_rows",
]
