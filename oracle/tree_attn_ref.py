"""CPU oracle for tree-draft verify attention -- test infrastructure only
(see the package docstring).

Sources: the review page "Speculative Decoding Meets Quantization" (ordoresearch.ai),
"The Compatibility Problem": tree-style verification holds several candidate
continuations and verifies them in parallel; the explainer page
"Speculative Decoding이란?" (dojself04.mycafe24.com), section 8 (Lookahead: a tree of
candidates A -> B, C, D checked by the large model at once) and section 10.1
(Medusa's "tree-based attention": candidate continuations arranged as a tree
and verified by the target in one pass).

Readings (the pages give no formula; each is listed in the design notes):
* One verify pass runs M draft tokens (the flattened tree) through attention.
  Draft token i attends to every position of the KV prefix (length L) and to
  the draft tokens marked in its ancestor mask (bit j of mask[i]: token i sees
  draft token j -- its ancestors and itself for a tree), never to the others.
* Scores are q . k * scale (scale = 1/sqrt(head dim)), softmax over the
  visible keys, output sum_k p_k v_k.  A token with no visible key outputs 0.
* Grouped-query attention: query head h reads key/value head h // (Hq / Hkv)
  (Llama-3-70B: 64 query heads, 8 key/value heads, head dim 128).

Everything here is float64.
"""
from __future__ import annotations

import numpy as np


def ancestor_masks(parents) -> np.ndarray:
    """uint64 masks of a tree given each draft token's parent (-1: a child of
    the prefix; parents precede children): bit j of mask[i] is set when j is
    i or an ancestor of i."""
    M = len(parents)
    if M > 64:
        raise ValueError("at most 64 draft tokens")
    masks = np.zeros(M, dtype=np.uint64)
    for i, p in enumerate(parents):
        if not -1 <= p < i:
            raise ValueError("parents must precede their children")
        masks[i] = (masks[p] if p >= 0 else np.uint64(0)) | np.uint64(1 << i)
    return masks


def tree_attention(q, k_cache, v_cache, k_draft, v_draft, masks, scale=None) -> np.ndarray:
    """q [M][Hq][D]; k_cache, v_cache [L][Hkv][D]; k_draft, v_draft [M][Hkv][D];
    masks [M] (uint64).  Returns [M][Hq][D] float64."""
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    kd = np.asarray(k_draft, dtype=np.float64)
    vd = np.asarray(v_draft, dtype=np.float64)
    M, Hq, D = q.shape
    Hkv = kc.shape[1] if kc.shape[0] else kd.shape[1]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((M, Hq, D))
    for i in range(M):
        vis = [j for j in range(M) if (int(masks[i]) >> j) & 1]
        for h in range(Hq):
            g = h // group
            keys = np.concatenate([kc[:, g, :], kd[vis, g, :]], axis=0)
            vals = np.concatenate([vc[:, g, :], vd[vis, g, :]], axis=0)
            if keys.shape[0] == 0:
                continue
            s = keys @ q[i, h] * scale
            p = np.exp(s - s.max())
            out[i, h] = (p / p.sum()) @ vals
    return out


def attention_weight_mass(q, k_cache, v_cache, k_draft, v_draft, masks, scale=None) -> np.ndarray:
    """sum_k p_k |v_k| per output element ([M][Hq][D]): the scale of the
    rounding a bf16 probability operand can introduce, used for the
    tolerance of the GPU comparison."""
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    kd = np.asarray(k_draft, dtype=np.float64)
    vd = np.asarray(v_draft, dtype=np.float64)
    M, Hq, D = q.shape
    Hkv = kc.shape[1] if kc.shape[0] else kd.shape[1]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((M, Hq, D))
    for i in range(M):
        vis = [j for j in range(M) if (int(masks[i]) >> j) & 1]
        for h in range(Hq):
            g = h // group
            keys = np.concatenate([kc[:, g, :], kd[vis, g, :]], axis=0)
            vals = np.concatenate([vc[:, g, :], vd[vis, g, :]], axis=0)
            if keys.shape[0] == 0:
                continue
            s = keys @ q[i, h] * scale
            p = np.exp(s - s.max())
            out[i, h] = (p / p.sum()) @ np.abs(vals)
    return out
