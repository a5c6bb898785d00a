"""CPU oracle for the acceptance step that follows the verify pass -- test
infrastructure only (see the package docstring).

Source: the explainer page "Speculative Decoding이란?" (dojself04.mycafe24.com),
section 3 (Leviathan et al., ICML 2023): Step 2, the target model scores every
drafted position in one forward pass; Step 3, the acceptance test
alpha = min(1, p(d)/q(d)), the drafted token d accepted when u < alpha with
u ~ U(0, 1); Step 4, at the first rejection the accepted prefix is kept and the
target model supplies the next token.  Section 5: greedy decoding gives the
same output as the target alone, and sampling the same distribution.  Section
6: the loop -- accept sequentially, at the first rejection sample from a
"corrected distribution".

Readings (the pages leave these open; each is listed in the design notes):
* Rows.  Verifying K drafted tokens yields K+1 rows of target logits: row j is
  the target's next-token distribution after the prefix and the first j
  drafted tokens (j = 0..K).  Draft row j (j < K) is the draft model's
  distribution from which drafted token j was drawn.
* p and q are the softmax of the logits (temperature 1).
* The corrected distribution is the residual normalise(max(0, p_j - q_j)) of
  the Leviathan et al. paper the page names; when all K drafted tokens are
  accepted the next token is drawn from p_K (the extra row).
* Greedy: drafted token j is accepted when it equals the first index of the
  maximum of target row j; the next token is the argmax of the first rejected
  row, or of row K.
* Drawing from a distribution r with a uniform u in [0, 1) is the inverse CDF:
  the smallest index t with r_0 + ... + r_t > u * (r_0 + ... + r_{V-1}).  The
  uniforms are inputs: u[j] for the test of drafted token j, u[K] for the
  final draw.

Everything here is float64.
"""
from __future__ import annotations

import numpy as np


def softmax64(logits) -> np.ndarray:
    """Row-wise softmax in float64."""
    x = np.asarray(logits, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def argmax_first(row) -> int:
    """First index of the maximum (the unique answer among equal maxima)."""
    return int(np.argmax(np.asarray(row)))


def inverse_cdf(r, u: float) -> int:
    """Smallest t with sum_{i<=t} r_i > u * sum_i r_i, for u in [0, 1)."""
    c = np.cumsum(np.asarray(r, dtype=np.float64))
    t = int(np.searchsorted(c, u * c[-1], side="right"))
    return min(t, len(c) - 1)


def accept_greedy(target_logits, draft_tokens):
    """Greedy acceptance: (number of drafted tokens accepted, next token)."""
    L = np.asarray(target_logits)
    K = len(draft_tokens)
    if L.shape[0] != K + 1:
        raise ValueError("K drafted tokens need K+1 target rows")
    for j in range(K):
        a = argmax_first(L[j])
        if int(draft_tokens[j]) != a:
            return j, a
    return K, argmax_first(L[K])


def accept_sampled(target_logits, draft_logits, draft_tokens, u):
    """Stochastic acceptance: (number of drafted tokens accepted, next token).

    u: K+1 uniforms in [0, 1)."""
    p = softmax64(target_logits)
    q = softmax64(draft_logits)
    K = len(draft_tokens)
    if p.shape[0] != K + 1 or q.shape[0] != K or len(u) != K + 1:
        raise ValueError("K drafted tokens need K+1 target rows, K draft rows and K+1 uniforms")
    for j in range(K):
        d = int(draft_tokens[j])
        alpha = 1.0 if q[j, d] == 0.0 else min(1.0, p[j, d] / q[j, d])
        if u[j] < alpha:
            continue
        return j, inverse_cdf(np.maximum(p[j] - q[j], 0.0), u[K])
    return K, inverse_cdf(p[K], u[K])


def decision_margins(target_logits, draft_logits, draft_tokens, u):
    """Distances of the stochastic decisions of accept_sampled from their
    boundaries (float64): |u_j - alpha_j| for every test taken, and for the
    final draw the distance of u*total from the nearest cumulative sum,
    relative to the total.  Used by tests to keep float32 rounding away from
    the decisions."""
    p = softmax64(target_logits)
    q = softmax64(draft_logits)
    K = len(draft_tokens)
    out = []
    row = None
    for j in range(K):
        d = int(draft_tokens[j])
        alpha = 1.0 if q[j, d] == 0.0 else min(1.0, p[j, d] / q[j, d])
        out.append(abs(u[j] - alpha))
        if not u[j] < alpha:
            row = np.maximum(p[j] - q[j], 0.0)
            break
    if row is None:
        row = p[K]
    c = np.cumsum(row)
    v = u[K] * c[-1]
    out.append(float(np.min(np.abs(c - v)) / c[-1]))
    return out
