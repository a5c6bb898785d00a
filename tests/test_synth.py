"""Checks of the seeded input generator (not of the method's arithmetic).

* Philox4x64-10 blocks equal numpy.random.Philox's (published generator);
* the fp16 and bf16 roundings equal numpy's / torch's round-to-nearest-even;
* the quantiser agrees with an independent numpy implementation of the same
  recipe and satisfies its data invariants (P7): s > 0, codes in [0, 15] and
  |w - (q - z) s| <= s/2 wherever no clamp was applied.
"""
import numpy as np
import pytest

import synth
from oracle import scales_to_f64, unpack_qweight, unpack_zeros


def test_philox_matches_numpy():
    for key0, block in [(0, 1), (1000, 5), (2 ** 63 + 17, 123456789)]:
        bg = np.random.Philox(key=np.array([key0, 0x57344131364D4131], dtype=np.uint64),
                              counter=np.array([block - 1, 0, 0, 0], dtype=np.uint64))
        assert np.array_equal(synth.philox_block(key0, 0x57344131364D4131, block), bg.random_raw(4))


def test_normals_are_standard_and_seeded():
    a = synth.normals(3, 1 << 20)
    assert abs(a.mean()) < 5e-3 and abs(a.std() - 1) < 5e-3
    assert np.array_equal(a[1000:1010], synth.normals(3, 10, start=1000))
    assert not np.array_equal(a[:16], synth.normals(4, 16))
    # tails behave like a Gaussian (P(|z| > 3) ~ 0.0027)
    frac = float(np.mean(np.abs(a) > 3))
    assert 0.002 < frac < 0.0034


def test_fp16_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.uniform(0, 0.02, 2000), rng.uniform(0, 1e-5, 500), 2.0 ** -np.arange(10, 26),
                           [0.0, 6.1e-5, 65504.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11]]).astype(np.float32)
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([synth.f32_to_f16_bits(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = synth.gen_x(3, 4096, seed_base=77)
    f = synth.normals(77, 4096)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(x[0], ref)


def _numpy_quantize(W, g=128):
    N, K = W.shape
    Wg = W.reshape(N, K // g, g)
    wmin = Wg.min(axis=2)
    wmax = Wg.max(axis=2)
    s16 = ((wmax - wmin) / np.float32(15)).astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(2.0 ** -14), s16)
    s = s16.astype(np.float32)
    z = np.clip(np.rint(-wmin / s), 0, 15)
    q = np.clip(np.rint(Wg / s[:, :, None]) + z[:, :, None], 0, 15)
    return q.reshape(N, K).astype(np.uint8), z.astype(np.uint8), s16


def test_quantizer_matches_independent_numpy_recipe():
    N, K = 64, 1024
    W = synth.weights_fp32(21, N, K)
    lin = synth.gen_linear(21, N, K)
    q, z, s16 = _numpy_quantize(W)
    assert np.array_equal(unpack_qweight(lin["qweight"]), q.T)
    assert np.array_equal(unpack_zeros(lin["zeros"]), z.T)
    assert np.array_equal(lin["scales"], s16.T.view(np.uint16))
    lin2 = synth.quantize(W)
    for k in lin:
        assert np.array_equal(lin[k], lin2[k])


def test_quantizer_invariants_and_degenerate_group():
    N, K, g = 16, 512, 128
    W = synth.weights_fp32(22, N, K)
    W[3, :128] = 0.0  # degenerate group: s -> 2^-14, q = z
    lin = synth.quantize(W)
    q = unpack_qweight(lin["qweight"]).T.astype(np.float64)
    z = unpack_zeros(lin["zeros"]).T.astype(np.float64)
    s = scales_to_f64(lin["scales"]).T
    assert np.all(s > 0) and s[3, 0] == 2.0 ** -14
    assert q.max() <= 15 and z.max() <= 15
    Wq = (q.reshape(N, K // g, g) - z[:, :, None]) * s[:, :, None]
    err = np.abs(W.reshape(N, K // g, g) - Wq)
    raw = np.rint(W.reshape(N, K // g, g) / s[:, :, None].astype(np.float32)) + z[:, :, None]
    unclipped = (raw >= 0) & (raw <= 15)
    assert np.all(err[unclipped] <= s[:, :, None].repeat(g, 2)[unclipped] * (0.5 + 1e-6))
    assert np.all(Wq[3, 0] == 0.0)


def test_thread_count_does_not_change_values():
    a = synth.gen_linear(5, 256, 256, nthreads=1)
    b = synth.gen_linear(5, 256, 256, nthreads=7)
    for k in a:
        assert np.array_equal(a[k], b[k])
