"""GPU parity of tree-draft verify attention (w4_tree_attention) against the
oracle (oracle/tree_attn_ref.py).

Inputs are bf16 (the oracle reads the same bf16 values in float64); the
kernel multiplies on bf16 MFMA with fp32 accumulation and rounds the softmax
probabilities to bf16 for the value product, so each output must lie within
1e-2 * sum_k p_k |v_k| of the oracle (a bf16 probability is off by at most
2^-9 of itself).  Cases: chains (sequence drafts), stars, random trees and
the page's A -> B, C, D tree; prefixes that end inside a 64-key chunk and on
its edge; the Llama-3-70B grouping (64 query heads over 8 key/value heads)
and other groupings; a token that sees nothing; one key split and the most
splits (M = 1 over 4096 and 12288 keys); repeatability, also with calls of
other shapes in between (the key splits' partial results share one
workspace, merged by a second launch), and under HIP graph replays.
"""
import numpy as np
import pytest

from oracle import ancestor_masks, attention_weight_mass, tree_attention

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

w4 = pytest.importorskip("speculative_decoding_verification_w4a16_amd")
DEV = "cuda:0"


def _bf16(rng, shape, sigma=1.0):
    """Random bf16 values: (bit patterns, the same values as float64)."""
    u = rng.normal(0.0, sigma, shape).astype(np.float32).view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return bits, (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _case(seed, M, L, Hq, Hkv, parents, sigma_q=1.0):
    rng = np.random.default_rng(seed)
    D = 128
    qb, q = _bf16(rng, (M, Hq, D), sigma_q)
    kcb, kc = _bf16(rng, (L, Hkv, D))
    vcb, vc = _bf16(rng, (L, Hkv, D))
    kdb, kd = _bf16(rng, (M, Hkv, D))
    vdb, vd = _bf16(rng, (M, Hkv, D))
    masks = ancestor_masks(parents) if parents is not None else np.zeros(M, np.uint64)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).to(DEV)
    out = w4.tree_attention(dev(qb), dev(kcb), dev(vcb), dev(kdb), dev(vdb),
                            torch.from_numpy(masks.view(np.int64)).to(DEV))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), (q, kc, vc, kd, vd, masks)


def _check(got, args, where):
    ref = tree_attention(*args)
    mass = attention_weight_mass(*args)
    err = np.abs(got - ref)
    bound = 1e-2 * mass + 1e-6
    assert np.all(err <= bound), (where, float(np.max(err / bound)))
    return float(np.max(err / bound))


def _random_tree(rng, M):
    return [-1] + [int(rng.integers(-1, i)) for i in range(1, M)]


@pytest.mark.parametrize("M,L,kind", [(1, 0, "chain"), (1, 200, "chain"), (5, 100, "chain"), (5, 128, "star"),
                                      (4, 61, "page"), (16, 1000, "tree"), (64, 64, "chain"), (64, 1000, "tree"),
                                      (64, 4096, "tree"), (1, 4096, "chain"), (8, 2047, "tree"),
                                      (2, 64 * 64 * 3, "chain"), (1, 1500, "chain")])
def test_tree_attention_matches_the_oracle(M, L, kind):
    rng = np.random.default_rng(M * 1000 + L)
    parents = {"chain": list(range(-1, M - 1)), "star": [-1] * M, "page": [-1, 0, 0, 0],
               "tree": _random_tree(rng, M)}[kind]
    got, args = _case(M + L, M, L, 64, 8, parents)
    _check(got, args, (M, L, kind))


@pytest.mark.parametrize("Hq,Hkv", [(16, 16), (32, 4), (8, 1)])
def test_other_head_groupings(Hq, Hkv):
    rng = np.random.default_rng(Hq + Hkv)
    got, args = _case(7, 9, 150, Hq, Hkv, _random_tree(rng, 9))
    _check(got, args, (Hq, Hkv))


def test_peaked_scores_and_unseen_tokens():
    # large queries make the softmax nearly one-hot: the online max must carry it
    got, args = _case(3, 12, 300, 64, 8, list(range(-1, 11)), sigma_q=8.0)
    _check(got, args, "peaked")
    # no prefix and empty masks: nothing to attend to, the output is 0
    got, args = _case(4, 6, 0, 64, 8, None)
    assert np.array_equal(got, np.zeros_like(got))


def test_repeatable():
    a, _ = _case(5, 33, 700, 64, 8, list(range(-1, 32)))
    b, _ = _case(5, 33, 700, 64, 8, list(range(-1, 32)))
    assert np.array_equal(a, b)


def test_repeatable_across_shapes():
    # the key splits' partial results go through one shared workspace and
    # are merged by a second launch; calls of other shapes in between (other
    # split counts and workspace extents) must not change the next result
    a, _ = _case(11, 1, 4096, 64, 8, [-1])
    _case(12, 64, 1000, 64, 8, list(range(-1, 63)))
    _case(13, 3, 30, 64, 8, [-1, 0, 1])
    b, args = _case(11, 1, 4096, 64, 8, [-1])
    assert np.array_equal(a, b)
    _check(b, args, "after other shapes")


def test_graph_replays_merge_every_time():
    # a captured call (the split kernel, then the merge launch) replays
    # correctly, also with the query changed between replays
    M, L, Hq, Hkv = 1, 4096, 64, 8
    rng = np.random.default_rng(4242)
    D = 128
    kcb, kc = _bf16(rng, (L, Hkv, D))
    vcb, vc = _bf16(rng, (L, Hkv, D))
    kdb, kd = _bf16(rng, (M, Hkv, D))
    vdb, vd = _bf16(rng, (M, Hkv, D))
    masks = ancestor_masks([-1])
    dev = lambda b: torch.from_numpy(b.view(np.int16)).to(DEV)
    qd = torch.empty((M, Hq, D), dtype=torch.int16, device=DEV)
    out = torch.empty((M, Hq, D), dtype=torch.float32, device=DEV)
    tens = [dev(kcb), dev(vcb), dev(kdb), dev(vdb), torch.from_numpy(masks.view(np.int64)).to(DEV)]
    qb0, _ = _bf16(rng, (M, Hq, D))
    qd.copy_(dev(qb0))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w4.tree_attention(qd, *tens, out=out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w4.tree_attention(qd, *tens, out=out)
    for rep in range(3):
        qb, q = _bf16(rng, (M, Hq, D))
        qd.copy_(dev(qb))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _check(out.cpu().numpy().astype(np.float64), (q, kc, vc, kd, vd, masks), ("graph replay", rep))
