"""Pins of the oracle's bf16 rounding (the bf16-output epilogue's reference)."""
import numpy as np
import pytest

import oracle
import synth


def _f(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


def test_representable_values_are_fixed_points():
    rng = np.random.default_rng(0)
    b = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32)
    b = b[(b & 0x7F80) != 0x7F80]  # finite
    assert np.array_equal(oracle.round_to_bf16(_f(b << 16)), b)


def test_ties_go_to_even():
    # 1 + 2^-8 lies halfway between 1 (even) and 1 + 2^-7 (odd): down
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even): up
    v = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), -(1 + 3 * 2.0 ** -8)], np.float32)
    assert list(oracle.round_to_bf16(v)) == [0x3F80, 0x3F82, 0xBF80, 0xBF82]


def test_nearest_and_half_ulp_bound():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-30, 30, 50000))).astype(np.float32)
    r = oracle.round_to_bf16(x).astype(np.uint32)
    back = _f(r << 16).astype(np.float64)
    ulp = np.abs(_f((r | np.uint32(1)) << 16).astype(np.float64) - _f((r & np.uint32(0xFFFE)) << 16))
    assert np.all(np.abs(back - x.astype(np.float64)) <= ulp / 2 * (1 + 1e-12))
    # monotone
    order = np.argsort(x)
    assert np.all(np.diff(back[order]) >= 0)


def test_overflow_threshold_rounds_to_infinity():
    # the largest bf16 is 0x7F7F; halfway to 2^128 (0x7F7F8000 as fp32) ties to even -> inf
    assert list(oracle.round_to_bf16(_f([0x7F7F7FFF, 0x7F7F8000, 0xFF7F8000]))) == [0x7F7F, 0x7F80, 0xFF80]


def test_agrees_with_the_input_generators_bit_formula():
    # an independent formulation: the integer round-half-even used to make bf16 inputs
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(100000) * 100).astype(np.float32)
    assert np.array_equal(oracle.round_to_bf16(x).astype(np.uint16), synth.f32_to_bf16_bits(x))


def test_rejects_non_finite():
    with pytest.raises(ValueError):
        oracle.round_to_bf16(np.array([np.inf], np.float32))
