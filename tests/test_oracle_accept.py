"""Pins of the acceptance-step oracle (oracle/accept_ref.py) to what the
explainer page "Speculative Decoding이란?" and probability fix, not to the
oracle's own formulas:

* the page's worked example (section 3 Steps 1 and 4) as a golden fixture;
* greedy identity (section 5): the emitted tokens are the target's own greedy
  decode, checked against a brute-force loop;
* losslessness (section 5): over random drafts and uniforms the first emitted
  token is distributed as the target's p, estimated by Monte Carlo;
* closed forms: draft equal to the target accepts everything; a one-hot
  draft is accepted with probability p(d) and its residual is p without d;
* the inverse-CDF draw on hand-computed cases;
* the decision margins (distance of each stochastic decision from its
  boundary) on a hand-computed three-token case and an all-accepted case.
"""
import json
import os

import numpy as np
import pytest

from oracle import accept_greedy, accept_sampled, argmax_first, decision_margins, inverse_cdf, softmax64

HERE = os.path.dirname(os.path.abspath(__file__))


def test_inverse_cdf_hand_cases():
    r = [0.2, 0.3, 0.5]
    assert [inverse_cdf(r, u) for u in (0.0, 0.19, 0.2, 0.49, 0.5, 0.999)] == [0, 0, 1, 1, 2, 2]
    assert inverse_cdf([0.0, 0.0, 3.0, 1.0], 0.0) == 2  # zero-probability tokens are never drawn
    assert inverse_cdf([0.0, 0.0, 3.0, 1.0], 0.75) == 3
    assert inverse_cdf([2.0, 2.0], 0.5) == 1  # unnormalised weights


def test_toy_example_from_the_page():
    g = json.load(open(os.path.join(HERE, "golden", "accept_toy_greedy.json")))
    vocab = g["vocab"]
    idx = {w: i for i, w in enumerate(vocab)}
    V = len(vocab)
    # target logits whose greedy continuation is the fixture's target_greedy
    rng = np.random.default_rng(0)
    L = rng.normal(0.0, 1.0, (len(g["target_greedy"]), V))
    for j, w in enumerate(g["target_greedy"]):
        L[j, idx[w]] = 5.0
    for case in g["cases"]:
        d = [idx[w] for w in case["draft"]]
        n, nxt = accept_greedy(L, d)
        emitted = [vocab[t] for t in d[:n]] + [vocab[nxt]]
        assert emitted == case["emitted"], case


def _brute_greedy(L, d):
    # the target's own greedy decode, position by position, plain Python
    out = []
    for j in range(len(d) + 1):
        row = list(L[j])
        best = max(row)
        out.append(row.index(best))
        if j < len(d) and d[j] != out[-1]:
            break
    return out


@pytest.mark.parametrize("seed", range(20))
def test_greedy_emits_the_targets_own_decode(seed):
    rng = np.random.default_rng(seed)
    V, K = 50, int(rng.integers(1, 8))
    L = rng.normal(0.0, 2.0, (K + 1, V))
    tgt = [int(np.argmax(L[j])) for j in range(K + 1)]
    # drafts that match the target for a random prefix, then differ
    k = int(rng.integers(0, K + 1))
    d = tgt[:k] + [int((t + 1 + rng.integers(0, V - 1)) % V) for t in tgt[k:K]]
    n, nxt = accept_greedy(L, d)
    assert n == k
    assert d[:n] + [nxt] == _brute_greedy(L, d)


def test_greedy_ties_take_the_first_index():
    L = np.zeros((2, 6))
    L[0, [1, 4]] = 3.0
    L[1, [2, 5]] = 1.0
    assert accept_greedy(L, [1]) == (1, 2)
    assert accept_greedy(L, [4]) == (0, 1)
    assert argmax_first([0.0, 2.0, 2.0]) == 1


def _first_token_distribution(p_logits, q_logits, K, trials, rng):
    V = p_logits.shape[1]
    q = softmax64(q_logits)
    counts = np.zeros(V)
    for _ in range(trials):
        d = [int(rng.choice(V, p=q[j])) for j in range(K)]
        u = rng.random(K + 1)
        n, nxt = accept_sampled(p_logits, q_logits, d, u)
        counts[d[0] if n >= 1 else nxt] += 1
    return counts / trials


@pytest.mark.parametrize("K", [1, 3])
def test_sampling_is_lossless(K):
    # section 5: the emitted token is distributed as the target's p (first row)
    rng = np.random.default_rng(11 + K)
    V = 5
    L = rng.normal(0.0, 1.0, (K + 1, V))
    Q = rng.normal(0.0, 1.0, (K, V))
    trials = 40000
    f = _first_token_distribution(L, Q, K, trials, rng)
    p0 = softmax64(L)[0]
    sigma = np.sqrt(p0 * (1 - p0) / trials)
    assert np.all(np.abs(f - p0) < 5 * sigma + 1e-3), (f, p0)
    # a wrong residual (plain p instead of max(0, p - q)) would break it
    q0 = softmax64(Q)[0]
    naive = np.minimum(p0, q0) + (1 - np.minimum(p0, q0).sum()) * p0
    assert np.max(np.abs(naive - p0)) > 10 * sigma.max()


def test_draft_equal_to_target_accepts_everything():
    rng = np.random.default_rng(5)
    K, V = 4, 30
    L = rng.normal(0.0, 2.0, (K + 1, V))
    for _ in range(50):
        d = [int(rng.integers(0, V)) for _ in range(K)]
        u = rng.random(K + 1)
        n, nxt = accept_sampled(L, L[:K], d, u)
        assert n == K
        assert nxt == inverse_cdf(softmax64(L)[K], u[K])  # the bonus token comes from row K


def test_one_hot_draft():
    # q = one-hot at d: alpha = p(d); the residual is p with d removed
    V, d = 6, 2
    L = np.log(np.array([[0.1, 0.2, 0.3, 0.15, 0.05, 0.2], [0.2] * 5 + [0.0001]]))
    Q = np.full((1, V), -1e3)
    Q[0, d] = 0.0
    assert accept_sampled(L, Q, [d], [0.29, 0.5])[0] == 1
    n, nxt = accept_sampled(L, Q, [d], [0.31, 0.0])
    assert n == 0 and nxt == 0
    r = np.array([0.1, 0.2, 0.0, 0.15, 0.05, 0.2]) / 0.7
    for u in (0.2, 0.5, 0.8, 0.99):
        assert accept_sampled(L, Q, [d], [0.9, u])[1] == int(np.searchsorted(np.cumsum(r), u, side="right"))


def test_decision_margins_cover_every_decision():
    rng = np.random.default_rng(3)
    K, V = 3, 40
    L = rng.normal(0.0, 1.0, (K + 1, V))
    Q = rng.normal(0.0, 1.0, (K, V))
    d = [int(rng.integers(0, V)) for _ in range(K)]
    u = rng.random(K + 1)
    m = decision_margins(L, Q, d, u)
    n, _ = accept_sampled(L, Q, d, u)
    assert len(m) == min(n + 1, K) + 1 and all(x >= 0 for x in m)


def _logits_of(probs):
    return np.log(np.asarray(probs, dtype=np.float64))


def test_decision_margins_hand_computed():
    # V = 4, K = 3; probabilities chosen so every decision is worked by hand
    p = [[0.4, 0.3, 0.2, 0.1],      # row 0: d = 0, alpha = min(1, 0.4 / 0.25) = 1
         [0.1, 0.2, 0.3, 0.4],      # row 1: d = 0, alpha = 0.1 / 0.5 = 0.2
         [0.25, 0.25, 0.25, 0.25],  # row 2: d = 1, alpha = 0.25 / 0.6 = 5/12
         [0.7, 0.1, 0.1, 0.1]]      # row 3: only drawn from when all three are kept
    q = [[0.25, 0.25, 0.25, 0.25],
         [0.5, 0.2, 0.2, 0.1],
         [0.1, 0.6, 0.2, 0.1]]
    d = [0, 0, 1]
    # u0 = 0.3 < 1 kept (margin 0.7); u1 = 0.15 < 0.2 kept (0.05); u2 = 0.5 >= 5/12
    # rejected (1/12).  Residual of row 2: max(0, p - q) = [0.15, 0, 0.05, 0.15],
    # total 0.35, cumulative [0.15, 0.15, 0.20, 0.35]; u3 * total = 0.21, nearest
    # cumulative sum 0.20: margin 0.01 / 0.35.
    u = [0.3, 0.15, 0.5, 0.6]
    m = decision_margins(_logits_of(p), _logits_of(q), d, u)
    assert accept_sampled(_logits_of(p), _logits_of(q), d, u) == (2, 3)
    assert np.allclose(m, [0.7, 0.05, 1.0 / 12.0, 0.01 / 0.35], rtol=1e-12, atol=1e-13), m
    # all three kept: the final draw is from row 3, cumulative [0.7, 0.8, 0.9, 1.0];
    # u3 = 0.84 lands 0.04 from 0.8 (total 1)
    u = [0.3, 0.15, 0.4, 0.84]
    m = decision_margins(_logits_of(p), _logits_of(q), d, u)
    assert accept_sampled(_logits_of(p), _logits_of(q), d, u) == (3, 2)
    assert np.allclose(m, [0.7, 0.05, 5.0 / 12.0 - 0.4, 0.04], rtol=1e-12, atol=1e-13), m
