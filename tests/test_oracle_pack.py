"""Pins of the oracle's unpacking (O1, O2) against independent packers.

The packers live in the input generator (``synth``, numpy and C); the
brute-force unpack below uses plain Python integers.  A wrong nibble order,
shift or axis in the oracle fails these."""
import numpy as np
import pytest

import synth
from oracle import unpack_qweight, unpack_zeros

pytestmark = pytest.mark.filterwarnings("ignore")


def _py_unpack_word(word: int):
    word &= 0xFFFFFFFF
    return [(word >> (4 * i)) & 0xF for i in range(8)]


def test_every_value_every_position():
    # q[8j+i, n] = v for every value v and nibble position i
    K, N = 8 * 16, 16
    q = np.zeros((K, N), np.uint8)
    for v in range(16):
        for i in range(8):
            q[8 * v + i, :] = v
    q[:, 1::2] = 15 - q[:, 1::2]
    assert np.array_equal(unpack_qweight(synth.pack_q(q)), q)
    z = np.arange(16 * 8, dtype=np.uint8).reshape(8, 16) % 16
    assert np.array_equal(unpack_zeros(synth.pack_z(z)), z)


def test_random_words_round_trip_including_sign_bit():
    rng = np.random.default_rng(1)
    w = rng.integers(-(2 ** 31), 2 ** 31, size=(64, 40), dtype=np.int64).astype(np.int32)
    w[0, 0] = -1
    w[0, 1] = -(2 ** 31)
    assert np.array_equal(synth.pack_q(unpack_qweight(w)), w)
    assert np.array_equal(synth.pack_z(unpack_zeros(w)), w)


def test_pure_python_unpack_agrees():
    rng = np.random.default_rng(2)
    w = rng.integers(-(2 ** 31), 2 ** 31, size=(5, 9), dtype=np.int64).astype(np.int32)
    q = unpack_qweight(w)
    z = unpack_zeros(w)
    for j in range(w.shape[0]):
        for n in range(w.shape[1]):
            nib = _py_unpack_word(int(w[j, n]))
            for i in range(8):
                assert q[8 * j + i, n] == nib[i]
                assert z[j, 8 * n + i] == nib[i]


def test_c_generator_packing_matches_numpy_packing():
    # the C quantiser's packed output, unpacked by the oracle and re-packed
    # by the numpy packer, is unchanged; and its codes are in range
    lin = synth.gen_linear(7, 64, 256)
    q = unpack_qweight(lin["qweight"])
    z = unpack_zeros(lin["zeros"])
    assert q.shape == (256, 64) and z.shape == (2, 64)
    assert np.array_equal(synth.pack_q(q), lin["qweight"])
    assert np.array_equal(synth.pack_z(z), lin["zeros"])
