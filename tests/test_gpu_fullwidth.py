"""GPU parity at full width and on the inputs the zero-mean tests miss.

* Every column of the seven Llama-3-70B-shaped linears (q, k, v, o, gate,
  up, down) against the oracle at M = 1 (plain decode), 5 (a sequence draft),
  16, 17 and 64 (tree drafts: the last one-block size, the first two-block
  size, four blocks) -- every tile, K split and row slice of the launch plans
  those shapes get.
* Activations with a non-zero mean (N(3, 1)) and with one outlier channel at
  +-3e4 placed where every weight of that channel is zero (q == z): the
  kernels accumulate x . (16 + q) and subtract (16 + z) * sum(x) per group,
  so these are the inputs where that cancellation is largest.  The contract
  must hold, and the error must stay inside the bound derived for the
  biased accumulation (fp32 roundings of partial sums of size
  (16 + q) * |x|, written out in check_biased_bound).
* Weight columns that are entirely zero (every group quantised from zeros:
  q = z = 0) give exactly 0, the only value the contract allows when
  sum_k |x w| = 0.
* Guard bytes before and after y: ragged N and M on every kernel path,
  fp32 and bf16 output, split and unsplit -- no store lands outside y.
"""
import numpy as np
import pytest

import synth
from oracle import bf16_bits_to_f64, linear64, linear64_gemm, round_to_bf16, unpack_qweight, unpack_zeros

from gpu_util import DEV, diagnostics, packed, run_linear, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

w4 = pytest.importorskip("speculative_decoding_verification_w4a16_amd")

FRO_MAX = 1e-5
FULL_M = (1, 5, 16, 17, 64)
COL_BLOCK = 4096  # oracle column block (bounded host memory)


def _check(y, Y, A, what, fro_max=FRO_MAX):
    d = diagnostics(y, Y, A)
    assert d["ok"], (what, d)
    if fro_max is not None:
        assert d["rel_fro"] < fro_max, (what, d)
    return d


@pytest.mark.parametrize("idx", range(len(synth.LAYER_LINEARS)))
def test_layer_linear_every_column(idx):
    name, N, K = synth.LAYER_LINEARS[idx]
    lin = synth.gen_linear(1000 + idx, N, K)
    pk = packed(lin, N, K)
    x = synth.gen_x(64, K)
    ys = {M: run_linear(x[:M], pk) for M in FULL_M}
    worst = 0.0
    for n0 in range(0, N, COL_BLOCK):
        n1 = min(N, n0 + COL_BLOCK)
        Y, A = linear64_gemm(x, lin["qweight"], lin["scales"], lin["zeros"], 128, n0, n1)
        for M in FULL_M:
            d = _check(ys[M][:, n0:n1], Y[:M], A[:M], (name, M, n0))
            worst = max(worst, d["worst"])
    print(f"{name}: every column at M in {FULL_M}, worst err/bound {worst:.2e}")


def check_biased_bound(y, x_bits, lin, K):
    """The error bound of the kernels' biased accumulation, per element:
    per group G the fp32 sums x . (16 + q) (at most 128 terms, then the
    group epilogue) and (16 + z) * sum(x) carry relative roundings of at most
    gamma = 132 * 2**-24 of sum_k |x_k| (16 + q_k) and of (16 + z) sum_k |x_k|,
    scaled by s_G; the scaled group terms then add up in fp32, with the K
    splits and cross-lane sums: at most (G + 64) roundings of sum_k |x w|.
    Asserts |y - Y64| <= that bound and returns the largest ratio."""
    q = unpack_qweight(lin["qweight"]).astype(np.float64)  # [K, N]
    z = unpack_zeros(lin["zeros"]).astype(np.float64)      # [G, N]
    s = lin["scales"].view(np.float16).astype(np.float64)  # [G, N]
    X = np.abs(bf16_bits_to_f64(x_bits))
    G = K // 128
    gamma = 132 * 2.0 ** -24
    bound = np.zeros((X.shape[0], q.shape[1]))
    for g in range(G):
        ks = slice(128 * g, 128 * (g + 1))
        Xa = X[:, ks]
        grp = Xa @ (16.0 + q[ks]) + Xa.sum(axis=1, keepdims=True) * (16.0 + z[g])
        bound += gamma * s[g] * grp
    Y, A = linear64(x_bits, lin["qweight"], lin["scales"], lin["zeros"])
    bound += (G + 64) * 2.0 ** -24 * A  # the sums of the scaled group terms
    err = np.abs(np.asarray(y, np.float64) - Y)
    assert np.all(err <= bound), float((err / bound).max())
    return float((err / bound).max()), Y, A


def _outlier_linear(seed, N, K, kstar):
    """A Gaussian linear whose input channel kstar has q == z in every column."""
    lin = synth.gen_linear(seed, N, K)
    q = unpack_qweight(lin["qweight"])
    z = unpack_zeros(lin["zeros"])
    q[kstar] = z[kstar // 128]
    return synth.pack_linear(q, z, lin["scales"])


@pytest.mark.parametrize("N,K", [(1024, 8192), (4096, 8192)])
def test_nonzero_mean_and_outlier_activations(N, K):
    # N(3, 1) activations; then N(0, 1) with channel kstar at +-3e4 where
    # every weight of that channel is zero; every kernel path (M = 1 GEMV,
    # 5 and 16 streaming or one-block LDS, 17 and 64 LDS with row slices on
    # the narrow linear)
    rng = np.random.default_rng(N + K)
    kstar = 3 * 128 + 77
    lin = _outlier_linear(600 + N, N, K, kstar)
    pk = packed(lin, N, K)
    x3 = synth.f32_to_bf16_bits(rng.normal(3.0, 1.0, (64, K)).astype(np.float32))
    xo = rng.normal(0.0, 1.0, (64, K)).astype(np.float32)
    xo[:, kstar] = np.where(np.arange(64) % 2 == 0, 3e4, -3e4)
    xo = synth.f32_to_bf16_bits(xo)
    for label, x in (("N(3,1)", x3), ("outlier at q == z", xo)):
        Y, A = linear64_gemm(x, lin["qweight"], lin["scales"], lin["zeros"], 128, 0, N)
        for M in FULL_M:
            y = run_linear(x[:M], pk)
            # the contract always; FRO_MAX for the mean-shifted input, the
            # derived bound of the biased accumulation for the outlier
            d = _check(y, Y[:M], A[:M], (label, N, M), fro_max=FRO_MAX if label == "N(3,1)" else None)
            ratio = None
            if label != "N(3,1)":
                ratio, _, _ = check_biased_bound(y, x[:M], lin, K)
            print(f"{label} N={N} M={M}: worst err/contract {d['worst']:.2e} rel_fro {d['rel_fro']:.2e}"
                  + (f" err/derived bound {ratio:.2e}" if ratio is not None else ""))


def test_all_zero_columns_are_exact_zeros():
    # weight columns quantised from zeros (every group: s = 2**-14, q = z = 0)
    # must give y = 0 exactly: sum_k |x w| = 0 leaves the contract no room
    N, K = 512, 4096
    W = synth.weights_fp32(77, N, K)
    zero_cols = [0, 5, 63, 64, 200, 511]
    W[zero_cols] = 0.0
    lin = synth.quantize(W)
    assert np.all(unpack_qweight(lin["qweight"])[:, zero_cols] == 0)
    pk = packed(lin, N, K)
    x = synth.gen_x(64, K, seed_base=1234)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    assert np.all(A[:, zero_cols] == 0)
    for M in (1, 5, 16, 17, 64):
        for splits in (0, 1, 3):
            y = run_linear(x[:M], pk, 0, splits)
            assert np.all(y[:, zero_cols] == 0.0), (M, splits)
            _check(y, Y[:M], A[:M], ("zero columns", M, splits))


def test_zero_columns_with_nonzero_zero_points_are_exact_zeros():
    # a symmetric quantiser stores zero weights as q = z = 8: columns (and
    # single groups) of such weights must still give exactly 0 (the contract
    # leaves no room where sum_k |x w| = 0), and the other columns the
    # contract; zero points 1..15 for the all-zero groups of one column
    N, K, g = 256, 4096, 128
    G = K // g
    rng = np.random.default_rng(97531)
    q = rng.integers(0, 16, size=(K, N))
    z = rng.integers(0, 16, size=(G, N))
    s = (np.float16(2.0 ** -7) * (0.5 + rng.random((G, N)))).astype(np.float16).view(np.uint16)
    zero_cols = [1, 70, 129, 250]
    z[:, zero_cols] = 8
    q[:, zero_cols] = 8
    z[:, 17] = (np.arange(G) % 15) + 1                 # zero point 1..15 per group
    q[:, 17] = np.repeat(z[:, 17], g)
    zero_cols.append(17)
    for gi in (0, 5, G - 1):                           # single all-zero groups in live columns
        q[gi * g:(gi + 1) * g, 40] = z[gi, 40]
    lin = synth.pack_linear(q, z, s)
    pk = packed(lin, N, K)
    x = synth.gen_x(64, K, seed_base=8642)
    x3 = synth.f32_to_bf16_bits(bf16_bits_to_f64(x).astype(np.float32) + 3.0)  # mean 3: large sum(x)
    for label, xx in (("N(0,1)", x), ("N(3,1)", x3)):
        Y, A = linear64(xx, lin["qweight"], lin["scales"], lin["zeros"])
        assert np.all(A[:, zero_cols] == 0)
        for M in FULL_M:
            for splits in (0, 1, 3):
                y = run_linear(xx[:M], pk, 0, splits)
                assert np.all(y[:, zero_cols] == 0.0), (label, M, splits, np.abs(y[:, zero_cols]).max())
                _check(y, Y[:M], A[:M], ("symmetric zeros", label, M, splits), fro_max=None)


def test_zero_negative_and_extreme_group_scales():
    # scales the quantiser never writes but a checkpoint may hold: +0 and -0
    # in single groups and over whole columns (those columns must give exactly
    # 0), negative scales, fp16 subnormals next to 65504 in the same column
    # (consecutive group scales 2**-24 and 65504 apart), on every kernel
    N, K, g = 256, 2048, 128
    G = K // g
    rng = np.random.default_rng(2468)
    q = rng.integers(0, 16, size=(K, N))
    z = rng.integers(0, 16, size=(G, N))
    s = (np.float16(2.0 ** -7) * (0.5 + rng.random((G, N)))).astype(np.float16).view(np.uint16)
    pick = rng.random((G, N))
    s[pick < 0.10] = 0x0000                           # +0
    s[(pick >= 0.10) & (pick < 0.15)] = 0x8000        # -0
    s[(pick >= 0.15) & (pick < 0.25)] |= 0x8000       # negative
    s[(pick >= 0.25) & (pick < 0.28)] = 0x0001        # smallest subnormal
    s[(pick >= 0.28) & (pick < 0.30)] = 0x7BFF        # largest finite
    zero_cols = [3, 64, 130, 255]
    s[:, zero_cols] = 0x0000
    s[::2, 200] = 0x8000                              # a column of alternating -0 and scale
    lin = synth.pack_linear(q, z, s)
    pk = packed(lin, N, K)
    x = synth.gen_x(64, K, seed_base=4321)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    assert np.all(A[:, zero_cols] == 0)
    for M in FULL_M:
        for splits in (0, 1, 3):
            y = run_linear(x[:M], pk, 0, splits)
            assert np.all(y[:, zero_cols] == 0.0), (M, splits)
            _check(y, Y[:M], A[:M], ("scales", M, splits), fro_max=None)


GUARD = 256  # bytes of guard on each side of y (keeps y 16-byte aligned)
PATTERN = 0xA5


@pytest.mark.parametrize("N", [8, 200, 1000, 27896])
def test_no_store_outside_y(N):
    K = 256
    lin = synth.gen_linear(300 + N, N, K)
    pk = packed(lin, N, K)
    x = synth.gen_x(64, K, seed_base=1500)
    xd = to_dev(x)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    for M in (1, 15, 17, 33, 63):
        kernels = [w4.W4_KERNEL_AUTO, w4.W4_KERNEL_MFMA] + ([w4.W4_KERNEL_GEMV] if M == 1 else [])
        for kern in kernels:
            for splits in (1, 2):
                for bf16 in (False, True):
                    esz = 2 if bf16 else 4
                    nbytes = M * N * esz
                    buf = torch.full((GUARD + nbytes + GUARD,), PATTERN, dtype=torch.uint8, device=DEV)
                    base = buf.data_ptr()
                    w4.w4a16_linear_tune(xd[:M], pk.qweight_t, pk.scales_t, pk.zeros_t, M, N, K, 128,
                                         base + GUARD, w4.W4_OUT_BF16 if bf16 else w4.W4_OUT_F32, kern, splits, 0)
                    torch.cuda.synchronize()
                    host = buf.cpu().numpy()
                    what = (N, M, kern, splits, bf16)
                    assert np.all(host[:GUARD] == PATTERN), what
                    assert np.all(host[GUARD + nbytes:] == PATTERN), what
                    y = host[GUARD:GUARD + nbytes]
                    if bf16:
                        yb = y.view(np.uint16).reshape(M, N)
                        yf = (yb.astype(np.uint32) << 16).view(np.float32)
                        # within the contract plus the bf16 rounding of the result
                        err = np.abs(yf.astype(np.float64) - Y[:M])
                        assert np.all(err <= 4e-3 * A[:M] * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(Y[:M])), what
                    else:
                        _check(y.view(np.float32).reshape(M, N), Y[:M], A[:M], what)


def test_bf16_output_is_the_rounded_fp32_output_on_guarded_buffers():
    # the same call with fp32 and bf16 output: bf16 = round_to_bf16(fp32)
    N, K, M = 1000, 1152, 33
    lin = synth.gen_linear(310, N, K)
    pk = packed(lin, N, K)
    x = to_dev(synth.gen_x(M, K, seed_base=1600))
    yf = w4.linear(x, pk)
    yb = w4.linear(x, pk, out_bf16=True)
    torch.cuda.synchronize()
    assert np.array_equal(yb.cpu().numpy().view(np.uint16), round_to_bf16(yf.cpu().numpy()).astype(np.uint16))
