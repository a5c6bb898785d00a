"""Planted mistakes in the oracle, each caught by at least one pin (CPU only).

Each case replaces one step of the oracle (module ``oracle.w4a16_ref``) with a
plausible wrong version -- a dropped zero-point term, a sign flip, nibbles in
the wrong order or shifted by one, a wrong group index, the scale applied per
column of the wrong group, a wrong bf16 decode, an absolute-value bound with
a signed factor -- and runs the pins of ``test_oracle_exact`` and
``test_oracle_invariants`` against it.  ``linear64`` looks its steps up in the
module at call time, so the planted step is what every pin that goes through
``linear64`` exercises.  The unmodified oracle passes the same pins in their
own modules.
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
    assert caught, f"no pin caught: {name}"
