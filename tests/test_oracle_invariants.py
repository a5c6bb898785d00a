"""Invariant pins of the oracle: linearity in x and row independence.

Verifying M draft tokens in one pass must give, row by row, what M
single-token passes give (ordoresearch.ai review, "Research Landscape": the
target checks the draft in one batched forward pass)."""
import numpy as np

import synth
from oracle import bf16_bits_to_f64, linear64
from oracle.w4a16_ref import _rows, _weights64


def _case(seed=11, M=6, K=512, N=96):
    lin = synth.gen_linear(seed, N, K)
    x = synth.gen_x(M, K, seed_base=500)
    return lin, x


def test_power_of_two_scaling_is_exact():
    lin, x = _case()
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    for e in (-3, 1, 4):
        xs = synth.f32_to_bf16_bits(bf16_bits_to_f64(x).astype(np.float32) * np.float32(2.0 ** e))
        Ye, Ae = linear64(xs, lin["qweight"], lin["scales"], lin["zeros"])
        assert np.array_equal(Ye, Y * 2.0 ** e)
        assert np.array_equal(Ae, A * 2.0 ** e)


def test_additivity_within_float64_bound():
    lin, x = _case(M=4)
    x1 = bf16_bits_to_f64(x[:2])
    x2 = bf16_bits_to_f64(x[2:])
    W64 = _weights64(lin["qweight"], lin["scales"], lin["zeros"], 128)
    K = W64.shape[0]
    # feed x1 + x2 as float64 rows directly (not representable in bf16)
    y12 = (x1 + x2) @ W64
    Y1, A1 = _rows(x[:2], W64)
    Y2, A2 = _rows(x[2:], W64)
    assert np.all(np.abs(y12 - (Y1 + Y2)) <= 2 * K * 2.0 ** -53 * (A1 + A2))


def test_m_tokens_equal_m_single_token_passes_bitwise():
    lin, x = _case(M=8)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    for m in range(x.shape[0]):
        y1, a1 = linear64(x[m:m + 1], lin["qweight"], lin["scales"], lin["zeros"])
        assert np.array_equal(y1[0], Y[m]) and np.array_equal(a1[0], A[m])
    # and a prefix of the rows gives the prefix of the result
    Y5, _ = linear64(x[:5], lin["qweight"], lin["scales"], lin["zeros"])
    assert np.array_equal(Y5, Y[:5])


def test_column_slice_matches_full():
    from oracle import linear64_columns

    lin, x = _case(M=3, N=128)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    Ys, As = linear64_columns(x, lin["qweight"], lin["scales"], lin["zeros"], 128, 40, 96)
    assert np.array_equal(Ys, Y[:, 40:96]) and np.array_equal(As, A[:, 40:96])


def test_matrix_product_form_matches_rows_and_the_exact_sum():
    # linear64_gemm is O6 as one matrix product per column block: the same
    # definition as linear64 in another float64 summation order.  Checked
    # against the row-by-row form and against the correctly rounded exact
    # sum (math.fsum of the exact products) within K * 2**-52 * A64, and exact
    # on one-hot rows (one nonzero product per element).
    import math

    from oracle import linear64_gemm

    lin, x = _case(seed=5, M=5, K=384, N=64)
    K = 384
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    Yg, Ag = linear64_gemm(x, lin["qweight"], lin["scales"], lin["zeros"], 128, 0, 64)
    bound = K * 2.0 ** -52 * A
    assert np.all(np.abs(Yg - Y) <= bound) and np.all(np.abs(Ag - A) <= K * 2.0 ** -52 * A)
    W64 = _weights64(lin["qweight"], lin["scales"], lin["zeros"], 128)
    X64 = bf16_bits_to_f64(x)
    for m in range(5):
        for n in range(0, 64, 7):
            exact = math.fsum(float(X64[m, k]) * float(W64[k, n]) for k in range(K))
            assert abs(Yg[m, n] - exact) <= K * 2.0 ** -53 * A[m, n]
    # a column block is the same block of the full product
    Yb, Ab = linear64_gemm(x, lin["qweight"], lin["scales"], lin["zeros"], 128, 16, 48)
    assert np.allclose(Yb, Yg[:, 16:48], rtol=0, atol=0) or np.all(np.abs(Yb - Yg[:, 16:48]) <= bound[:, 16:48])
    e = synth.f32_to_bf16_bits(np.eye(K, dtype=np.float32)[[0, 7, 127, 128, 383]])
    Ye, _ = linear64_gemm(e, lin["qweight"], lin["scales"], lin["zeros"], 128, 0, 64)
    assert np.array_equal(Ye, W64[[0, 7, 127, 128, 383]])
