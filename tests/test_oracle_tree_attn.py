"""Pins of the tree-attention oracle (oracle/tree_attn_ref.py) to properties
that the pages and the mathematics fix, not to its own formula:

* the ancestor masks of hand-built trees, among them the page's Lookahead
  tree A -> B, C, D (explainer page "Speculative Decoding이란?", section 8);
* tree verification equals verifying each root-to-token path as a sequence:
  checked against a brute-force loop (math.exp, plain lists) on tiny sizes;
* closed forms: one visible key returns its value; identical keys average
  the visible values;
* invariants: a shift of every key by the same vector, and a permutation of
  the prefix, leave the output unchanged; query heads read the key/value head
  h // (Hq / Hkv);
* the weight mass sum_k p_k |v_k| (the tolerance scale of the GPU checks):
  against a brute-force loop, one visible key (= |v|), identical keys (= the
  mean of |v|), non-negative values (= the attention output itself) and the
  triangle inequality |output| <= mass.
"""
import math

import numpy as np
import pytest

from oracle import ancestor_masks, attention_weight_mass, tree_attention


def test_ancestor_masks_of_hand_built_trees():
    assert [int(m) for m in ancestor_masks([-1, 0, 1])] == [0b1, 0b11, 0b111]  # a chain: causal
    assert [int(m) for m in ancestor_masks([-1, -1, -1])] == [0b1, 0b10, 0b100]  # siblings only see themselves
    # the page's Lookahead tree: A with children B, C, D
    assert [int(m) for m in ancestor_masks([-1, 0, 0, 0])] == [0b1, 0b11, 0b101, 0b1001]
    assert int(ancestor_masks(list(range(-1, 63)))[63]) == (1 << 64) - 1
    with pytest.raises(ValueError):
        ancestor_masks([-1, 2, 0])


def _brute_path_attention(q, keys, vals, scale):
    s = [scale * sum(a * b for a, b in zip(k, q)) for k in keys]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    z = sum(w)
    return [sum(wi * v[d] for wi, v in zip(w, vals)) / z for d in range(len(vals[0]))]


def _rand(rng, M, L, Hq=4, Hkv=2, D=8):
    return (rng.normal(size=(M, Hq, D)), rng.normal(size=(L, Hkv, D)), rng.normal(size=(L, Hkv, D)),
            rng.normal(size=(M, Hkv, D)), rng.normal(size=(M, Hkv, D)))


@pytest.mark.parametrize("seed", range(6))
def test_tree_equals_each_path_as_a_sequence(seed):
    rng = np.random.default_rng(seed)
    M, L, Hq, Hkv, D = 7, 5, 4, 2, 8
    parents = [-1] + [int(rng.integers(-1, i)) for i in range(1, M)]
    q, kc, vc, kd, vd = _rand(rng, M, L, Hq, Hkv, D)
    out = tree_attention(q, kc, vc, kd, vd, ancestor_masks(parents))
    for i in range(M):
        path = []
        j = i
        while j >= 0:
            path.append(j)
            j = parents[j]
        path.reverse()
        for h in range(Hq):
            g = h // (Hq // Hkv)
            keys = [list(kc[t, g]) for t in range(L)] + [list(kd[t, g]) for t in path]
            vals = [list(vc[t, g]) for t in range(L)] + [list(vd[t, g]) for t in path]
            exp = _brute_path_attention(list(q[i, h]), keys, vals, 1 / math.sqrt(D))
            assert np.allclose(out[i, h], exp, rtol=1e-12, atol=1e-12)


def test_one_visible_key_and_identical_keys():
    rng = np.random.default_rng(1)
    M, Hq, Hkv, D = 5, 4, 2, 8
    q, _, _, kd, vd = _rand(rng, M, 0, Hq, Hkv, D)
    kc = np.zeros((0, Hkv, D))
    out = tree_attention(q, kc, kc, kd, vd, ancestor_masks([-1] * M))  # each token sees only itself
    for i in range(M):
        for h in range(Hq):
            assert np.array_equal(out[i, h], vd[i, h // 2])
    # identical keys everywhere: the output is the plain mean of the visible values
    L = 6
    kc = np.ones((L, Hkv, D))
    vc = rng.normal(size=(L, Hkv, D))
    kd1 = np.ones((M, Hkv, D))
    masks = ancestor_masks([-1, 0, 1, 1, 3])
    out = tree_attention(q, kc, vc, kd1, vd, masks)
    for i in range(M):
        vis = [j for j in range(M) if (int(masks[i]) >> j) & 1]
        for h in range(Hq):
            g = h // 2
            mean = (vc[:, g].sum(0) + vd[vis, g].sum(0)) / (L + len(vis))
            assert np.allclose(out[i, h], mean, rtol=1e-12, atol=1e-12)


def test_invariances_and_head_grouping():
    rng = np.random.default_rng(2)
    M, L, Hq, Hkv, D = 6, 9, 8, 2, 16
    q, kc, vc, kd, vd = _rand(rng, M, L, Hq, Hkv, D)
    masks = ancestor_masks([-1, 0, 0, 1, 2, 2])
    base = tree_attention(q, kc, vc, kd, vd, masks)
    # shifting every key of a head by one vector shifts every score of a query equally
    u = rng.normal(size=(1, Hkv, D))
    assert np.allclose(tree_attention(q, kc + u, vc, kd + u, vd, masks), base, rtol=1e-10, atol=1e-10)
    perm = rng.permutation(L)
    assert np.allclose(tree_attention(q, kc[perm], vc[perm], kd, vd, masks), base, rtol=1e-10, atol=1e-10)
    # equal queries: heads 0..3 share key/value head 0 and agree; head 4 reads head 1 and differs
    q2 = q.copy()
    q2[:, :, :] = q[:, :1, :]
    out = tree_attention(q2, kc, vc, kd, vd, masks)
    assert np.allclose(out[:, 1], out[:, 0]) and np.allclose(out[:, 3], out[:, 0])
    assert not np.allclose(out[:, 4], out[:, 0])


def _brute_path_mass(q, keys, vals, scale):
    s = [scale * sum(a * b for a, b in zip(k, q)) for k in keys]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    z = sum(w)
    return [sum(wi * abs(v[d]) for wi, v in zip(w, vals)) / z for d in range(len(vals[0]))]


@pytest.mark.parametrize("seed", range(3))
def test_weight_mass_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    M, L, Hq, Hkv, D = 6, 4, 4, 2, 8
    parents = [-1] + [int(rng.integers(-1, i)) for i in range(1, M)]
    masks = ancestor_masks(parents)
    q, kc, vc, kd, vd = _rand(rng, M, L, Hq, Hkv, D)
    mass = attention_weight_mass(q, kc, vc, kd, vd, masks)
    for i in range(M):
        vis = [j for j in range(M) if (int(masks[i]) >> j) & 1]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            keys = [list(kc[t, g]) for t in range(L)] + [list(kd[t, g]) for t in vis]
            vals = [list(vc[t, g]) for t in range(L)] + [list(vd[t, g]) for t in vis]
            exp = _brute_path_mass(list(q[i, h]), keys, vals, 1 / math.sqrt(D))
            assert np.allclose(mass[i, h], exp, rtol=1e-12, atol=1e-12)


def test_weight_mass_closed_forms():
    rng = np.random.default_rng(7)
    M, Hq, Hkv, D = 5, 4, 2, 8
    q, _, _, kd, vd = _rand(rng, M, 0, Hq, Hkv, D)
    empty = np.zeros((0, Hkv, D))
    # one visible key (each token sees only itself, no prefix): the mass is |v|
    mass = attention_weight_mass(q, empty, empty, kd, vd, ancestor_masks([-1] * M))
    for i in range(M):
        for h in range(Hq):
            assert np.array_equal(mass[i, h], np.abs(vd[i, h // 2]))
    # identical keys: every visible key has weight 1/n, the mass is the mean of |v|
    L = 6
    kc = np.ones((L, Hkv, D))
    vc = rng.normal(size=(L, Hkv, D))
    kd1 = np.ones((M, Hkv, D))
    masks = ancestor_masks([-1, 0, 1, 1, 3])
    mass = attention_weight_mass(q, kc, vc, kd1, vd, masks)
    for i in range(M):
        vis = [j for j in range(M) if (int(masks[i]) >> j) & 1]
        for h in range(Hq):
            g = h // 2
            mean_abs = (np.abs(vc[:, g]).sum(0) + np.abs(vd[vis, g]).sum(0)) / (L + len(vis))
            assert np.allclose(mass[i, h], mean_abs, rtol=1e-12, atol=1e-12)
    # random keys: |output| <= mass, with equality when every value is >= 0
    q, kc, vc, kd, vd = _rand(rng, M, 7, Hq, Hkv, D)
    masks = ancestor_masks([-1, 0, 0, 2, 1])
    out = tree_attention(q, kc, vc, kd, vd, masks)
    mass = attention_weight_mass(q, kc, vc, kd, vd, masks)
    assert np.all(np.abs(out) <= mass * (1 + 1e-12) + 1e-15)
    assert np.any(np.abs(out) < 0.5 * mass)  # signed values cancel; the mass does not
    out_pos = tree_attention(q, kc, np.abs(vc), kd, np.abs(vd), masks)
    mass_pos = attention_weight_mass(q, kc, np.abs(vc), kd, np.abs(vd), masks)
    assert np.allclose(out_pos, mass_pos, rtol=1e-12, atol=1e-14)
    # a token that sees nothing has zero mass
    mass0 = attention_weight_mass(q[:1], empty, empty, kd[:1], vd[:1], np.zeros(1, dtype=np.uint64))
    assert np.array_equal(mass0, np.zeros_like(mass0))
