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
splits (M = 1 over 4096 and 12288 keys); both ways of merging the key
splits (a second launch; the last workgroup of each row tile, counted in on
an arrival counter that it sets back to zero); repeatability, also with
calls of other shapes and the other merge in between (the partial results
and the counters share one workspace), and under HIP graph replays.
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


MERGES = (w4.TREE_MERGE_LAUNCH, w4.TREE_MERGE_LAST)


def _case(seed, M, L, Hq, Hkv, parents, sigma_q=1.0, merge=w4.TREE_MERGE_AUTO):
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
                            torch.from_numpy(masks.view(np.int64)).to(DEV), merge=merge)
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


@pytest.mark.parametrize("merge", MERGES)
@pytest.mark.parametrize("M,L,kind", [(1, 0, "chain"), (1, 200, "chain"), (5, 100, "chain"), (5, 128, "star"),
                                      (4, 61, "page"), (16, 1000, "tree"), (64, 64, "chain"), (64, 1000, "tree"),
                                      (64, 4096, "tree"), (1, 4096, "chain"), (8, 2047, "tree"),
                                      (2, 64 * 64 * 3, "chain"), (1, 1500, "chain"), (17, 3000, "tree"),
                                      (5, 4096, "chain")])
def test_tree_attention_matches_the_oracle(M, L, kind, merge):
    rng = np.random.default_rng(M * 1000 + L)
    parents = {"chain": list(range(-1, M - 1)), "star": [-1] * M, "page": [-1, 0, 0, 0],
               "tree": _random_tree(rng, M)}[kind]
    got, args = _case(M + L, M, L, 64, 8, parents, merge=merge)
    _check(got, args, (M, L, kind, merge))


@pytest.mark.parametrize("merge", MERGES)
@pytest.mark.parametrize("Hq,Hkv", [(16, 16), (32, 4), (8, 1)])
def test_other_head_groupings(Hq, Hkv, merge):
    rng = np.random.default_rng(Hq + Hkv)
    got, args = _case(7, 9, 150, Hq, Hkv, _random_tree(rng, 9), merge=merge)
    _check(got, args, (Hq, Hkv, merge))


@pytest.mark.parametrize("M,L", [(1, 1024), (1, 4096), (2, 500), (5, 4096)])
def test_the_default_merge_matches_the_forced_one(M, L):
    # the default takes the merge the plan names (the last workgroup for
    # small tiles, a second launch otherwise): bit for bit the same output
    splits, used = w4.w4_tree_attention_plan(M, L, 64, 8)
    assert splits > 1 and used in MERGES
    a, args = _case(30 + M, M, L, 64, 8, list(range(-1, M - 1)))
    b, _ = _case(30 + M, M, L, 64, 8, list(range(-1, M - 1)), merge=used)
    assert np.array_equal(a, b), (M, L, used)
    _check(a, args, (M, L, "default"))
    # one split: nothing to merge
    assert w4.w4_tree_attention_plan(1, 0, 64, 8) == (1, w4.TREE_MERGE_AUTO)


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


@pytest.mark.parametrize("merge", MERGES)
def test_repeatable_across_shapes(merge):
    # the key splits' partial results and the arrival counters go through
    # one shared workspace; calls of other shapes and of the other merge in
    # between (other split counts, tile counts and workspace extents) must
    # not change the next result: every call leaves the counters at zero
    other = MERGES[1 - MERGES.index(merge)]
    a, _ = _case(11, 1, 4096, 64, 8, [-1], merge=merge)
    _case(12, 64, 1000, 64, 8, list(range(-1, 63)), merge=other)
    _case(13, 3, 30, 64, 8, [-1, 0, 1], merge=merge)
    _case(14, 64, 4096, 64, 8, list(range(-1, 63)), merge=merge)
    _case(15, 17, 3000, 64, 8, list(range(-1, 16)), merge=other)
    b, args = _case(11, 1, 4096, 64, 8, [-1], merge=merge)
    assert np.array_equal(a, b)
    _check(b, args, ("after other shapes", merge))


@pytest.mark.parametrize("merge", MERGES)
def test_graph_replays_merge_every_time(merge):
    # a captured call (the split kernel and the merge launch, or the split
    # kernel alone with its arrival counters) replays correctly, also with
    # the query changed between replays
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
        w4.tree_attention(qd, *tens, out=out, stream=s, merge=merge)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w4.tree_attention(qd, *tens, out=out, merge=merge)
    for rep in range(3):
        qb, q = _bf16(rng, (M, Hq, D))
        qd.copy_(dev(qb))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _check(out.cpu().numpy().astype(np.float64), (q, kc, vc, kd, vd, masks), ("graph replay", rep, merge))
        # an eager call of another shape between replays
        _case(20 + rep, 5, 700, 64, 8, list(range(-1, 4)), merge=merge)


def test_interleaved_graph_replays_of_shapes_sharing_the_counters():
    # three captured calls of different shapes -- two merged in the last
    # workgroup of each tile (different tile and split counts), one by a
    # second launch -- replayed interleaved: each replay must match the
    # oracle, so no call leaves an arrival counter another one reads
    shapes = [(1, 1024), (2, 500), (64, 1000)]
    D, Hq, Hkv = 128, 64, 8
    rng = np.random.default_rng(777)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).to(DEV)
    cases = []
    for M, L in shapes:
        qb, q = _bf16(rng, (M, Hq, D))
        kcb, kc = _bf16(rng, (L, Hkv, D))
        vcb, vc = _bf16(rng, (L, Hkv, D))
        kdb, kd = _bf16(rng, (M, Hkv, D))
        vdb, vd = _bf16(rng, (M, Hkv, D))
        masks = ancestor_masks(_random_tree(rng, M))
        tens = [dev(qb), dev(kcb), dev(vcb), dev(kdb), dev(vdb), torch.from_numpy(masks.view(np.int64)).to(DEV)]
        out = torch.empty((M, Hq, D), dtype=torch.float32, device=DEV)
        cases.append((tens, out, (q, kc, vc, kd, vd, masks)))
    used = [w4.w4_tree_attention_plan(M, L, Hq, Hkv)[1] for M, L in shapes]
    assert used == [w4.TREE_MERGE_LAST, w4.TREE_MERGE_LAST, w4.TREE_MERGE_LAUNCH], used
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for tens, out, _ in cases:
            w4.tree_attention(*tens, out=out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graphs = []
    for tens, out, _ in cases:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            w4.tree_attention(*tens, out=out)
        graphs.append(g)
    for step, i in enumerate([0, 1, 2, 0, 1, 0, 2, 1]):
        tens, out, args = cases[i]
        out.fill_(float("nan"))
        graphs[i].replay()
        torch.cuda.synchronize()
        _check(out.cpu().numpy().astype(np.float64), args, ("interleaved replay", step, shapes[i]))
