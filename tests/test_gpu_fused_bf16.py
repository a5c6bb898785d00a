"""GPU parity of the fused-projection / bf16-epilogue follow-up.

* bf16 output: w4a16_linear_out(W4_OUT_BF16) equals, bit for bit, the
  oracle's round-to-nearest-even of the fp32 output of the same kernel and
  split count (every kernel variant, split and unsplit K, ragged N), and
  the rounded values meet the contract plus half a bf16 ulp;
* fused projections: the tile layout of a column concatenation is the
  concatenation of the parts' layouts (bit-exact, against w4_repack of the
  concatenated canonical arrays), and the fused qkv (N = 10240) and
  gate|up (N = 57344) linears meet the contract on every part's sampled
  columns at the verify sizes.
"""
import numpy as np
import pytest

import synth
from oracle import check_contract, linear64, linear64_columns, round_to_bf16

from gpu_util import DEV, packed, to_dev, torch_mod

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

w4 = pytest.importorskip("speculative_decoding_verification_w4a16_amd")


def _run(x_bits, pk, out_bf16, kernel=0, splits=0):
    xd = to_dev(x_bits)
    y = w4.linear(xd, pk, kernel=kernel, splits=splits, out_bf16=out_bf16)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("N,K", [(256, 512), (200, 384), (1000, 1152)])
@pytest.mark.parametrize("M,kernel", [(1, 1), (1, 2), (5, 0), (16, 0), (17, 0), (33, 0), (64, 0)])
def test_bf16_output_is_the_rounded_fp32_output(N, K, M, kernel):
    lin = synth.gen_linear(77, N, K)
    pk = packed(lin, N, K)
    x = synth.gen_x(M, K, seed_base=500)
    G = K // 128
    for splits in sorted({1, min(3, G), G}):
        y32 = _run(x, pk, False, kernel, splits)
        yb = _run(x, pk, True, kernel, splits).view(np.uint16)
        assert yb.shape == (M, N)
        exp = round_to_bf16(y32).astype(np.uint16)
        assert np.array_equal(yb, exp), (N, K, M, kernel, splits)
        # and the rounded result still meets the contract, widened by half a bf16 ulp of |y|
        Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
        yv = (yb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.all(np.abs(yv - Y) <= 4e-3 * A + np.abs(Y) * 2.0 ** -8 + 1e-30)


def test_bf16_output_degenerate_calls():
    N, K = 256, 512
    lin = synth.gen_linear(3, N, K)
    pk = packed(lin, N, K)
    y = torch.full((2, N), 0x3F80, dtype=torch.int16, device=DEV)
    w4.w4a16_linear_out(to_dev(synth.gen_x(2, K)), pk.qweight_t, pk.scales_t, pk.zeros_t, 2, N, 0, 128, y,
                        w4.W4_OUT_BF16)
    torch.cuda.synchronize()
    assert int(y.abs().sum()) == 0  # K = 0 writes bf16 zeros over all M*N outputs
    with pytest.raises(w4.W4Error):
        w4.w4a16_linear_out(0x1000, 0x2000, 0x3000, 0x4000, 2, N, K, 128, 0x100000, 7)


FUSED = {"qkv": ("q", "k", "v"), "gate_up": ("gate", "up")}


@pytest.fixture(scope="module")
def parts():
    out = {}
    for idx, (name, N, K) in enumerate(synth.LAYER_LINEARS):
        if name in ("q", "k", "v", "gate", "up"):
            out[name] = (synth.gen_linear(1000 + idx, N, K), N, K)
    return out


@pytest.mark.parametrize("fused", list(FUSED))
def test_concatenated_tile_layout_is_bit_exact(parts, fused):
    names = FUSED[fused]
    K = parts[names[0]][2]
    lins = [parts[n][0] for n in names]
    Ns = [parts[n][1] for n in names]
    cat = {"qweight": np.concatenate([l["qweight"] for l in lins], axis=1),
           "scales": np.concatenate([l["scales"] for l in lins], axis=1),
           "zeros": np.concatenate([l["zeros"] for l in lins], axis=1)}
    whole = packed(cat, sum(Ns), K)
    glued = w4.concat_packed([packed(l, n, K) for l, n in zip(lins, Ns)])
    assert glued.N == whole.N == sum(Ns)
    for a, b in ((whole.qweight_t, glued.qweight_t), (whole.scales_t, glued.scales_t),
                 (whole.zeros_t, glued.zeros_t)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("fused", list(FUSED))
def test_fused_projection_contract(parts, fused):
    names = FUSED[fused]
    K = parts[names[0]][2]
    pk = w4.concat_packed([packed(parts[n][0], parts[n][1], K) for n in names])
    x = synth.gen_x(64, K)
    rng = np.random.default_rng(99)
    checks = []
    n0 = 0
    for n in names:
        lin, N, _ = parts[n]
        a = int(rng.integers(0, N // 64)) * 64
        Y, A = linear64_columns(x, lin["qweight"], lin["scales"], lin["zeros"], 128, a, a + 64)
        checks.append((n0 + a, Y, A, n))
        n0 += N
    for M in (1, 5, 16, 17, 48, 64):
        y = _run(x[:M], pk, False)
        yb = _run(x[:M], pk, True).view(np.uint16)
        assert np.array_equal(yb, round_to_bf16(y).astype(np.uint16))
        for c0, Y, A, n in checks:
            ok, worst = check_contract(y[:, c0:c0 + 64], Y[:M], A[:M])
            assert ok, (fused, n, M, worst)
