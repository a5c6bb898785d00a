"""Pins of the oracle's arithmetic (O3-O7) against exact sums and closed forms.

Each expected value here is computed from the *constructed* codes, zeros and
scales in plain Python (``fractions``/``math.fsum``), not from the oracle's
own unpacking, so a dropped term, a wrong sign, a wrong group index or a
transposed operand in the oracle fails at least one test."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import bf16_bits_to_f64, check_contract, dequant64, linear64, scales_to_f64, unpack_qweight, \
    unpack_zeros

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.txt")


def _random_case(rng, M, K, N, g=128):
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    z = rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)
    s = (rng.uniform(1e-3, 1e-2, size=(K // g, N))).astype(np.float16)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    lin = synth.pack_linear(q, z, s.view(np.uint16))
    return q, z, s, x, lin


def _bf16_to_float(b):
    return float(np.array([int(b) << 16], np.uint32).view(np.float32)[0])


def test_golden_worked_example():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            m, n, y = line.split()
            rows[(int(m), int(n))] = float(y)
    K, N, g = 256, 8, 128
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    q = ((k + n) % 16).astype(np.uint8)
    G = np.arange(K // g)[:, None]
    z = ((3 * G + n) % 16).astype(np.uint8)
    s = (2.0 ** -(G + 1) * (n + 1)).astype(np.float16)
    x = np.stack([np.ones(K, np.float32), np.where(np.arange(K) % 2 == 0, 1.0, -1.0).astype(np.float32)])
    lin = synth.pack_linear(q, z, s.view(np.uint16))
    Y, A = linear64(synth.f32_to_bf16_bits(x), lin["qweight"], lin["scales"], lin["zeros"], g)
    for (mm, nn), v in rows.items():
        assert Y[mm, nn] == v, (mm, nn, Y[mm, nn], v)


def test_dequant_exact_in_float64_and_fp32():
    # P2: (q - z) * s is exact: it equals the float32 product widened, and the
    # exact rational product
    rng = np.random.default_rng(3)
    q, z, s, x, lin = _random_case(rng, 1, 256, 64)
    W64 = dequant64(unpack_qweight(lin["qweight"]), unpack_zeros(lin["zeros"]), scales_to_f64(lin["scales"]), 128)
    W32 = ((q.astype(np.float32).reshape(2, 128, 64) - z.astype(np.float32)[:, None, :])
           * s.astype(np.float32)[:, None, :]).reshape(256, 64)
    assert np.array_equal(W64, W32.astype(np.float64))
    for kk, nn in [(0, 0), (127, 5), (128, 63), (255, 31)]:
        exact = (int(q[kk, nn]) - int(z[kk // 128, nn])) * Fraction(float(s[kk // 128, nn]))
        assert Fraction(W64[kk, nn]) == exact


def test_bf16_decode_exact():
    bits = np.array([0x0000, 0x3F80, 0xBF80, 0x4300, 0x0001, 0x7F7F, 0xC2F7], np.uint16)
    exp = [0.0, 1.0, -1.0, 128.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, -123.5]
    assert list(bf16_bits_to_f64(bits)) == exp


def test_brute_force_fsum_tiny_config():
    # P3: on the tiny linear shape (K=512, N=256, M=4) the oracle equals the
    # correctly rounded exact sum within K * 2^-53 * sum|x w|
    rng = np.random.default_rng(4)
    M, K, N, g = 4, 512, 256, 128
    q, z, s, x, lin = _random_case(rng, M, K, N, g)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"], g)
    xf = [[_bf16_to_float(b) for b in row] for row in x]
    sf = s.astype(np.float64).tolist()
    ql = q.tolist()
    zl = z.tolist()
    for m in range(M):
        for n in range(0, N, 7):
            terms = [xf[m][k] * ((ql[k][n] - zl[k // g][n]) * sf[k // g][n]) for k in range(K)]
            exact = math.fsum(terms)
            absum = math.fsum(abs(t) for t in terms)
            assert abs(Y[m, n] - exact) <= K * 2.0 ** -53 * absum
            assert A[m, n] == pytest.approx(absum, rel=1e-12)


def test_q_equals_z_gives_exact_zero():
    rng = np.random.default_rng(5)
    K, N, g = 384, 32, 128
    z = rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)
    q = np.repeat(z, g, axis=0)
    s = np.full((K // g, N), 0.01, np.float16)
    lin = synth.pack_linear(q, z, s.view(np.uint16))
    x = synth.f32_to_bf16_bits(rng.standard_normal((3, K)).astype(np.float32))
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"], g)
    assert np.all(Y == 0.0) and np.all(A == 0.0)


def test_one_hot_rows_pick_weight_rows():
    # x = e_k picks the dequantised weight row k, computed here from the
    # constructed codes (nibble positions 0..7, group edges, first/last k)
    rng = np.random.default_rng(6)
    K, N, g = 384, 48, 128
    q, z, s, _, lin = _random_case(rng, 1, K, N, g)
    ks = [0, 1, 2, 3, 4, 5, 6, 7, 127, 128, 129, 255, 256, 383]
    x = np.zeros((len(ks), K), np.float32)
    for i, kk in enumerate(ks):
        x[i, kk] = 1.0
    Y, _ = linear64(synth.f32_to_bf16_bits(x), lin["qweight"], lin["scales"], lin["zeros"], g)
    for i, kk in enumerate(ks):
        exp = (q[kk].astype(np.float64) - z[kk // g].astype(np.float64)) * s[kk // g].astype(np.float64)
        assert np.array_equal(Y[i], exp)


def test_integer_gemm_special_case():
    # s = 1 and z = 8 with small-integer x: the oracle is an integer GEMM,
    # checked against numpy's int64 matmul (textbook)
    rng = np.random.default_rng(7)
    M, K, N, g = 5, 256, 40, 128
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    z = np.full((K // g, N), 8, np.uint8)
    s = np.ones((K // g, N), np.float16)
    xi = rng.integers(-9, 10, size=(M, K))
    lin = synth.pack_linear(q, z, s.view(np.uint16))
    Y, _ = linear64(synth.f32_to_bf16_bits(xi.astype(np.float32)), lin["qweight"], lin["scales"], lin["zeros"], g)
    exp = xi.astype(np.int64) @ (q.astype(np.int64) - 8)
    assert np.array_equal(Y, exp.astype(np.float64))


def test_all_ones_closed_form():
    # x = 1: y[n] = sum_G s[G, n] * sum_{k in G} (q[k, n] - z[G, n]), in integers
    rng = np.random.default_rng(8)
    K, N, g = 512, 24, 128
    q, z, s, _, lin = _random_case(rng, 1, K, N, g)
    x = synth.f32_to_bf16_bits(np.ones((1, K), np.float32))
    Y, _ = linear64(x, lin["qweight"], lin["scales"], lin["zeros"], g)
    for n in range(N):
        tot = Fraction(0)
        for G in range(K // g):
            d = int(q[G * g:(G + 1) * g, n].astype(np.int64).sum()) - g * int(z[G, n])
            tot += Fraction(float(s[G, n])) * d
        assert Y[0, n] == pytest.approx(float(tot), rel=1e-15, abs=1e-300)


def test_single_group_reduces_to_scaled_dot():
    # K = g: y = s * (x . (q - z)), an fsum-exact dot
    rng = np.random.default_rng(9)
    K, N, g = 128, 16, 128
    q, z, s, x, lin = _random_case(rng, 2, K, N, g)
    Y, _ = linear64(x, lin["qweight"], lin["scales"], lin["zeros"], g)
    for m in range(2):
        xs = [_bf16_to_float(b) for b in x[m]]
        for n in range(N):
            dot = math.fsum(xs[k] * (int(q[k, n]) - int(z[0, n])) for k in range(K))
            assert Y[m, n] == pytest.approx(float(s[0, n]) * dot, rel=1e-14, abs=1e-300)


def test_contract_check_semantics():
    Y = np.array([[1.0, 0.0, -2.0]])
    A = np.array([[10.0, 0.0, 5.0]])
    bound = 4e-3 * A
    ok, worst = check_contract(Y + np.array([[0.999, 0.0, -0.5]]) * bound, Y, A)
    assert ok and worst == pytest.approx(0.999, rel=1e-9)
    ok, _ = check_contract(Y + np.array([[1.001, 0.0, 0.0]]) * bound, Y, A)
    assert not ok
    ok, worst = check_contract(Y + np.array([[0.0, 1e-30, 0.0]]), Y, A)
    assert not ok and worst == float("inf")
