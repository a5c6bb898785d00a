"""Planted mistakes in the oracle, each caught by at least one pin (CPU only).

Each case replaces one step of an oracle with a
plausible wrong version -- a dropped zero-point term, a sign flip, nibbles in
the wrong order or shifted by one, a wrong group index, the scale applied per
column of the wrong group, a wrong bf16 decode, an absolute-value bound with
a signed factor; in the acceptance step the wrong tie-break, draw, count,
test or residual, and decision margins measured from the wrong boundary; in
tree attention an ignored mask, a missing scale or a wrong head grouping, and a
weight mass without the probabilities, with signed values or with
unnormalised weights -- and runs the pins against it until one fails.  The
steps are replaced where the pins look them up (``linear64`` finds its own
steps in ``oracle.w4a16_ref`` at call time).  The unmodified oracles pass the
same pins in their own modules.
"""
import numpy as np
import pytest

import oracle.w4a16_ref as ref
import test_oracle_exact as exact
import test_oracle_invariants as invariants

_orig_unpack_qweight = ref.unpack_qweight
_orig_dequant64 = ref.dequant64


def _unpack_nibbles(qweight, order):
    w = np.ascontiguousarray(qweight).view(np.uint32)
    kw, n = w.shape
    out = np.empty((kw, 8, n), np.uint8)
    for i in range(8):
        out[:, i, :] = (w >> np.uint32(4 * order(i))) & np.uint32(0xF)
    return out.reshape(kw * 8, n)


def _dequant_no_zero(q, z, s64, group):
    K, N = q.shape
    G = K // group
    return (q.astype(np.float64).reshape(G, group, N) * s64.reshape(G, 1, N)).reshape(K, N)


def _dequant_sign_flipped(q, z, s64, group):
    return -_orig_dequant64(q, z, s64, group)


def _dequant_group_of_k_mod_g(q, z, s64, group):
    # scale and zero of group k % G instead of k // group
    K, N = q.shape
    G = K // group
    gi = np.arange(K) % G
    return (q.astype(np.float64) - z[gi].astype(np.float64)) * s64[gi]


def _dequant_last_group_scale(q, z, s64, group):
    # every group scaled by the last group's scale
    K, N = q.shape
    G = K // group
    d = q.astype(np.int16).reshape(G, group, N) - z.astype(np.int16).reshape(G, 1, N)
    return (d.astype(np.float64) * s64[-1].reshape(1, 1, N)).reshape(K, N)


def _bf16_shift_15(x_bits):
    u = np.ascontiguousarray(x_bits).view(np.uint16).astype(np.uint32) << np.uint32(15)
    return u.view(np.float32).astype(np.float64)


def _rows_signed_bound(x_bits, W64):
    X64 = ref.bf16_bits_to_f64(np.atleast_2d(x_bits))
    return X64 @ W64, np.abs(X64) @ W64


def _rows_transposed_x(x_bits, W64):
    X64 = ref.bf16_bits_to_f64(np.atleast_2d(x_bits))
    # the rows of x reversed along k (a transposed or mis-strided operand)
    X64 = X64[:, ::-1]
    return X64 @ W64, np.abs(X64) @ np.abs(W64)


MUTANTS = {
    "dropped zero-point term": ("dequant64", _dequant_no_zero),
    "sign of the weight flipped": ("dequant64", _dequant_sign_flipped),
    "group index k % G": ("dequant64", _dequant_group_of_k_mod_g),
    "one scale for every group": ("dequant64", _dequant_last_group_scale),
    "nibbles in reverse order": ("unpack_qweight", lambda w: _unpack_nibbles(w, lambda i: 7 - i)),
    "nibble index shifted by one": ("unpack_qweight", lambda w: _unpack_nibbles(w, lambda i: (i + 1) % 8)),
    "bf16 decoded with a 15-bit shift": ("bf16_bits_to_f64", _bf16_shift_15),
    "bound with a signed weight": ("_rows", _rows_signed_bound),
    "activations reversed along k": ("_rows", _rows_transposed_x),
}

PINS = [
    exact.test_golden_worked_example,
    exact.test_brute_force_fsum_tiny_config,
    exact.test_q_equals_z_gives_exact_zero,
    exact.test_one_hot_rows_pick_weight_rows,
    exact.test_integer_gemm_special_case,
    exact.test_all_ones_closed_form,
    exact.test_single_group_reduces_to_scaled_dot,
    invariants.test_power_of_two_scaling_is_exact,
    invariants.test_additivity_within_float64_bound,
    invariants.test_m_tokens_equal_m_single_token_passes_bitwise,
]


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ref, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # an assertion, or a shape error the mistake causes
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught: {name}"


# ---------------------------------------------------------------------------
# the acceptance step and tree attention oracles
# ---------------------------------------------------------------------------

import functools  # noqa: E402

import oracle.accept_ref as acc  # noqa: E402
import test_oracle_accept as accept_pins  # noqa: E402
import test_oracle_tree_attn as tree_pins  # noqa: E402

_orig_inverse_cdf = acc.inverse_cdf


def _argmax_last(row):
    r = np.asarray(row)
    return int(len(r) - 1 - np.argmax(r[::-1]))


def _inverse_cdf_ge(r, u):
    c = np.cumsum(np.asarray(r, dtype=np.float64))
    return min(int(np.searchsorted(c, u * c[-1], side="left")), len(c) - 1)


def _greedy_off_by_one(target_logits, draft_tokens):
    L = np.asarray(target_logits)
    K = len(draft_tokens)
    for j in range(K):
        a = acc.argmax_first(L[j])
        if int(draft_tokens[j]) != a:
            return j + 1, a
    return K, acc.argmax_first(L[K])


def _sampled_variant(kind, target_logits, draft_logits, draft_tokens, u):
    p, q = acc.softmax64(target_logits), acc.softmax64(draft_logits)
    K = len(draft_tokens)
    for j in range(K):
        d = int(draft_tokens[j])
        alpha = 1.0 if q[j, d] == 0.0 else min(1.0, p[j, d] / q[j, d])
        keep = u[j] > alpha if kind == "flipped test" else u[j] < alpha
        if keep:
            continue
        residual = p[j] if kind == "target row at rejection" else np.maximum(p[j] - q[j], 0.0)
        return j, _orig_inverse_cdf(residual, u[K])
    return K, _orig_inverse_cdf(p[K] if kind != "draft row at the end" else q[K - 1], u[K])


def _tree_variant(kind, q, k_cache, v_cache, k_draft, v_draft, masks, scale=None):
    q = np.asarray(q, dtype=np.float64)
    kc, vc = np.asarray(k_cache, dtype=np.float64), np.asarray(v_cache, dtype=np.float64)
    kd, vd = np.asarray(k_draft, dtype=np.float64), np.asarray(v_draft, dtype=np.float64)
    M, Hq, D = q.shape
    Hkv = kc.shape[1] if kc.shape[0] else kd.shape[1]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 if kind == "no 1/sqrt(d) scale" else 1.0 / np.sqrt(D)
    out = np.zeros((M, Hq, D))
    for i in range(M):
        if kind == "mask ignored":
            vis = list(range(M))
        elif kind == "own token not seen":
            vis = [j for j in range(M) if j != i and (int(masks[i]) >> j) & 1]
        else:
            vis = [j for j in range(M) if (int(masks[i]) >> j) & 1]
        for h in range(Hq):
            g = h % Hkv if kind == "head h reads h % Hkv" else h // group
            keys = np.concatenate([kc[:, g, :], kd[vis, g, :]], axis=0)
            vals = np.concatenate([vc[:, g, :], vd[vis, g, :]], axis=0)
            if keys.shape[0] == 0:
                continue
            s = keys @ q[i, h] * scale
            p = np.exp(s - s.max())
            out[i, h] = (p / p.sum()) @ vals
    return out


def _mass_variant(kind, q, k_cache, v_cache, k_draft, v_draft, masks, scale=None):
    q = np.asarray(q, dtype=np.float64)
    kc, vc = np.asarray(k_cache, dtype=np.float64), np.asarray(v_cache, dtype=np.float64)
    kd, vd = np.asarray(k_draft, dtype=np.float64), np.asarray(v_draft, dtype=np.float64)
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
            if kind == "sum |v| without p":
                out[i, h] = np.abs(vals).sum(axis=0)
            elif kind == "signed v":
                out[i, h] = (p / p.sum()) @ vals
            else:  # unnormalised weights
                out[i, h] = p @ np.abs(vals)
    return out


def _margins_variant(kind, target_logits, draft_logits, draft_tokens, u):
    p, q = acc.softmax64(target_logits), acc.softmax64(draft_logits)
    K = len(draft_tokens)
    out, row = [], None
    for j in range(K):
        d = int(draft_tokens[j])
        ratio = 1.0 if q[j, d] == 0.0 else p[j, d] / q[j, d]
        alpha = min(1.0, ratio)
        out.append(abs(u[j] - (ratio if kind == "uncapped ratio" else alpha)))
        if not u[j] < alpha:
            row = p[j] if kind == "target row" else np.maximum(p[j] - q[j], 0.0)
            break
    if row is None:
        row = p[K]
    c = np.cumsum(row)
    v = u[K] if kind == "u, not u * total" else u[K] * c[-1]
    out.append(float(np.min(np.abs(c - v)) / c[-1]))
    return out


# (module the pins look the name up in, name, mutant)
MUTANTS_F = {
    "greedy: last index of equal maxima": [(acc, "argmax_first", _argmax_last),
                                           (accept_pins, "argmax_first", _argmax_last)],
    "draw: cumulative weight >= u total": [(acc, "inverse_cdf", _inverse_cdf_ge),
                                           (accept_pins, "inverse_cdf", _inverse_cdf_ge)],
    "greedy: one token too many accepted": [(accept_pins, "accept_greedy", _greedy_off_by_one)],
    "sampled: acceptance test flipped": [(accept_pins, "accept_sampled",
                                          functools.partial(_sampled_variant, "flipped test"))],
    "sampled: target row, not the residual": [(accept_pins, "accept_sampled",
                                               functools.partial(_sampled_variant, "target row at rejection"))],
    "sampled: last draft row at the end": [(accept_pins, "accept_sampled",
                                            functools.partial(_sampled_variant, "draft row at the end"))],
    "tree: mask ignored": [(tree_pins, "tree_attention", functools.partial(_tree_variant, "mask ignored"))],
    "tree: own token not seen": [(tree_pins, "tree_attention",
                                  functools.partial(_tree_variant, "own token not seen"))],
    "tree: no 1/sqrt(d) scale": [(tree_pins, "tree_attention",
                                  functools.partial(_tree_variant, "no 1/sqrt(d) scale"))],
    "tree: head h reads h % Hkv": [(tree_pins, "tree_attention",
                                    functools.partial(_tree_variant, "head h reads h % Hkv"))],
    "mass: sum |v| without p": [(tree_pins, "attention_weight_mass",
                                 functools.partial(_mass_variant, "sum |v| without p"))],
    "mass: signed v": [(tree_pins, "attention_weight_mass", functools.partial(_mass_variant, "signed v"))],
    "mass: unnormalised weights": [(tree_pins, "attention_weight_mass",
                                    functools.partial(_mass_variant, "unnormalised weights"))],
    "margins: test measured from p/q, not min(1, p/q)": [
        (accept_pins, "decision_margins", functools.partial(_margins_variant, "uncapped ratio"))],
    "margins: final draw measured from u, not u * total": [
        (accept_pins, "decision_margins", functools.partial(_margins_variant, "u, not u * total"))],
    "margins: final draw on the target row, not the residual": [
        (accept_pins, "decision_margins", functools.partial(_margins_variant, "target row"))],
}

PINS_F = [
    accept_pins.test_inverse_cdf_hand_cases,
    accept_pins.test_toy_example_from_the_page,
    functools.partial(accept_pins.test_greedy_emits_the_targets_own_decode, 0),
    functools.partial(accept_pins.test_greedy_emits_the_targets_own_decode, 7),
    accept_pins.test_greedy_ties_take_the_first_index,
    functools.partial(accept_pins.test_sampling_is_lossless, 1),
    functools.partial(accept_pins.test_sampling_is_lossless, 3),
    accept_pins.test_draft_equal_to_target_accepts_everything,
    accept_pins.test_one_hot_draft,
    functools.partial(tree_pins.test_tree_equals_each_path_as_a_sequence, 0),
    functools.partial(tree_pins.test_tree_equals_each_path_as_a_sequence, 3),
    tree_pins.test_one_visible_key_and_identical_keys,
    tree_pins.test_invariances_and_head_grouping,
    functools.partial(tree_pins.test_weight_mass_brute_force, 0),
    tree_pins.test_weight_mass_closed_forms,
    accept_pins.test_decision_margins_hand_computed,
]


@pytest.mark.parametrize("name", list(MUTANTS_F))
def test_planted_mistake_in_accept_or_tree_oracle_fails_a_pin(name, monkeypatch):
    for module, attr, fn in MUTANTS_F[name]:
        monkeypatch.setattr(module, attr, fn)
    caught = []
    for pin in PINS_F:
        try:
            pin()
        except Exception:
            caught.append(pin)
            break
    assert caught, f"no pin caught: {name}"
