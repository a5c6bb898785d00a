"""GPU parity of the acceptance step (w4_accept_greedy / w4_accept_sample)
against the oracle (oracle/accept_ref.py).

Greedy decisions are exact integer comparisons of fp32 logits, so they must
match bit for bit, ties included (first index of the maximum, also across
the slices the kernel splits a row into).  The sampled decisions compare
fp32 quantities with uniforms; the inputs are drawn so that every decision
stays clear of its boundary by far more than fp32 rounding (the oracle's
decision_margins), and then (accepted count, next token) must match exactly.
Sizes: the Llama-3 vocabulary (128256) and small ones, K from 0 to 64.
"""
import numpy as np
import pytest

from oracle import accept_greedy, accept_sampled, decision_margins, softmax64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

w4 = pytest.importorskip("speculative_decoding_verification_w4a16_amd")
DEV = "cuda:0"
VOCAB = 128256


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).to(DEV)


def _greedy(L, d):
    out = w4.accept(_dev(L, np.float32), _dev(d, np.int32))
    torch.cuda.synchronize()
    return tuple(int(v) for v in out.cpu())


def _sampled(L, Q, d, u):
    out = w4.accept(_dev(L, np.float32), _dev(d, np.int32), _dev(Q, np.float32), _dev(u, np.float32))
    torch.cuda.synchronize()
    return tuple(int(v) for v in out.cpu())


@pytest.mark.parametrize("V", [128, 1000, VOCAB])
@pytest.mark.parametrize("K", [0, 1, 4, 16, 63, 64])
def test_greedy_matches_the_oracle(V, K):
    rng = np.random.default_rng(100 + K + V)
    L = rng.normal(0.0, 2.0, (K + 1, V)).astype(np.float32)
    tgt = L.argmax(axis=1)
    for k in sorted({0, K // 2, K}):
        d = np.concatenate([tgt[:k], (tgt[k:K] + 1 + rng.integers(0, V - 1, K - k)) % V]).astype(np.int32)
        assert _greedy(L, d) == accept_greedy(L, d), (V, K, k)


def test_greedy_ties_and_out_of_range_drafts():
    V, K = VOCAB, 3
    L = np.zeros((K + 1, V), np.float32)
    # equal maxima in different slices of a row: the first index wins
    L[0, [90000, 7, 128000]] = 5.0
    L[1, [64000, 64001]] = 2.0
    L[2, [VOCAB - 1]] = 1.0
    L[3, [3, 1]] = 9.0
    assert _greedy(L, np.array([7, 64000, VOCAB - 1], np.int32)) == accept_greedy(L, [7, 64000, VOCAB - 1]) == (3, 1)
    assert _greedy(L, np.array([90000, 0, 0], np.int32)) == (0, 7)
    assert _greedy(L, np.array([7, -1, 0], np.int32)) == (1, 64000)  # out-of-range draft: rejected
    assert _greedy(L, np.array([7, 64000, VOCAB], np.int32)) == (2, VOCAB - 1)


def _sampled_case(rng, K, V, noise, offset=0.0):
    """Target and draft logits, drafted tokens drawn from the draft's q, and
    uniforms whose decisions all clear their boundaries."""
    L = (rng.normal(0.0, 2.0, (K + 1, V)) + offset).astype(np.float32)
    Q = (L[:K] + rng.normal(0.0, noise, (K, V))).astype(np.float32)
    q = softmax64(Q)
    d = np.array([rng.choice(V, p=q[j]) for j in range(K)], np.int32)
    for _ in range(200):
        u = rng.random(K + 1).astype(np.float32)
        m = decision_margins(L, Q, d, u.astype(np.float64))
        if min(m[:-1], default=1.0) > 1e-5 and m[-1] > 2e-6:
            return L, Q, d, u
    raise AssertionError("no well-separated uniforms found")


@pytest.mark.parametrize("V", [1000, VOCAB])
@pytest.mark.parametrize("K", [1, 4, 16, 64])
def test_sampled_matches_the_oracle(V, K):
    rng = np.random.default_rng(7 * K + V)
    seen = set()
    for trial in range(6):
        L, Q, d, u = _sampled_case(rng, K, V, noise=0.7 if trial % 2 else 2.0)
        exp = accept_sampled(L, Q, d, u.astype(np.float64))
        assert _sampled(L, Q, d, u) == exp, (V, K, trial)
        seen.add(exp[0] == K)
    assert seen  # both outcomes usually occur; correctness is checked either way


def test_sampled_bonus_row_and_one_hot_draft():
    rng = np.random.default_rng(21)
    V, K = VOCAB, 4
    # draft equal to the target: every token accepted, the next one drawn from row K
    L = rng.normal(0.0, 2.0, (K + 1, V)).astype(np.float32)
    d = np.array([rng.choice(V, p=softmax64(L[:K])[j]) for j in range(K)], np.int32)
    for _ in range(5):
        u = rng.random(K + 1).astype(np.float32)
        if decision_margins(L, L[:K], d, u.astype(np.float64))[-1] > 2e-6:
            got = _sampled(L, L[:K], d, u)
            assert got[0] == K and got == accept_sampled(L, L[:K], d, u.astype(np.float64))
    # a one-hot draft: accepted iff u < p(d); the residual is p without d
    Q = np.full((K, V), -1e4, np.float32)
    Q[np.arange(K), d] = 0.0
    p = softmax64(L)
    for u0 in (0.5 * p[0, d[0]], 1.5 * p[0, d[0]] + 1e-6):
        for ur in np.linspace(0.05, 0.95, 19):
            u = np.array([u0, 0.9, 0.9, 0.9, ur], np.float32)
            m = decision_margins(L, Q, d, u.astype(np.float64))
            if min(m[:-1]) > 1e-5 and m[-1] > 2e-6:
                break
        assert _sampled(L, Q, d, u) == accept_sampled(L, Q, d, u.astype(np.float64))


def test_large_logit_offsets_and_determinism():
    rng = np.random.default_rng(33)
    K, V = 8, VOCAB
    L, Q, d, u = _sampled_case(rng, K, V, noise=1.0, offset=3000.0)
    a = _sampled(L, Q, d, u)
    assert a == accept_sampled(L, Q, d, u.astype(np.float64))
    assert a == _sampled(L, Q, d, u)  # fixed reduction order: repeatable
    assert _greedy(L, d) == accept_greedy(L, d)


def test_errors_before_any_launch():
    with pytest.raises(w4.W4Error):
        w4.w4_accept_greedy(0x1000, 0x2000, 65, 1024, 0x3000, stream=0)


@pytest.mark.parametrize("V", [1000, VOCAB])
def test_final_draw_at_the_top_of_the_distribution(V):
    # u just below 1 puts u * total at (or, after fp32 rounding, past) the last
    # inclusive sum: the draw must still return the last token with weight.
    # The last token carries a large weight, so the oracle's float64 decision
    # is the same token, far from any boundary.  Also u = 0: the first token
    # with weight; and the draft equal to the target (all kept, row K drawn).
    rng = np.random.default_rng(44 + V)
    K = 3
    L = rng.normal(0.0, 1.0, (K + 1, V)).astype(np.float32)
    L[:, V - 1] = 8.0
    L[:, V - 2] = -1e4  # the second-to-last token has no weight (exp underflows to 0 in fp32 and float64)
    L[:, 0] = 6.0
    d = np.array([V - 1] * K, np.int32)
    top = np.float32(1.0) - np.float32(2.0 ** -24)
    for uK in (top, np.float32(0.0)):
        u = np.array([0.5] * K + [uK], np.float32)
        exp = accept_sampled(L, L[:K], d, u.astype(np.float64))
        assert exp == (K, V - 1 if uK > 0 else 0)
        for _ in range(3):  # the same answer on every run
            assert _sampled(L, L[:K], d, u) == exp, (V, float(uK))
    # rejected at token 0 (the draft puts almost all its mass there): the residual
    # max(0, p - q) keeps the last token, where the draft has less mass than the
    # target, and the draw at u -> 1 returns it
    Q = L[:K].copy()
    Q[0, V - 1] = 6.0
    Q[0, 0] = 20.0
    d0 = np.array([0, V - 1, V - 1], np.int32)
    u = np.array([0.99, 0.5, 0.5, top], np.float32)
    exp = accept_sampled(L, Q, d0, u.astype(np.float64))
    assert exp == (0, V - 1)
    assert _sampled(L, Q, d0, u) == exp
