"""GPU parity of the K-splitting workgroups of the M <= 16 kernels.

A workgroup of kwaves waves streams one 64-column chunk, its waves taking
contiguous parts of the groups and summing their results in LDS; with
splits > 1 the sum goes to the split-K workspace instead of y.  Every forced
(kwaves, splits) pair meets the contract against the oracle on shapes that
span several chunks, a ragged N and group counts that do not divide evenly,
its bf16 output is the rounded fp32 output of the same plan, and results do
not depend on which decomposition ran beyond the contract.
"""
import numpy as np
import pytest

import synth
from oracle import check_contract, linear64, round_to_bf16

from gpu_util import packed, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

w4 = pytest.importorskip("speculative_decoding_verification_w4a16_amd")


def _run(x_bits, pk, kwaves, splits, out_bf16=False, kernel=0):
    y = w4.linear(to_dev(x_bits), pk, kernel=kernel, splits=splits, kwaves=kwaves, out_bf16=out_bf16)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("N,K", [(256, 1024), (1000, 1152), (200, 384), (640, 2816)])
@pytest.mark.parametrize("M,kernel", [(1, 1), (1, 2), (2, 0), (5, 0), (16, 0)])
def test_k_splitting_workgroups_meet_the_contract(N, K, M, kernel):
    lin = synth.gen_linear(91, N, K)
    pk = packed(lin, N, K)
    x = synth.gen_x(M, K, seed_base=700)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    G = K // 128
    for kwaves in (2, 4, 8):
        for splits in sorted({1, 2, min(3, G)}):
            plan = w4.w4a16_plan(M, N, K, kernel=kernel, splits=splits, kwaves=kwaves)
            assert plan["kwaves"] <= kwaves
            y = _run(x, pk, kwaves, splits, kernel=kernel)
            ok, worst = check_contract(y, Y, A)
            assert ok, (N, K, M, kernel, kwaves, splits, plan, worst)


@pytest.mark.parametrize("M", [15, 16])
def test_forced_waves_keep_wide_m16_on_the_streaming_kernel(M):
    # Left to the planner, M = 15 and 16 on 4096 or more columns run the LDS
    # kernel; a forced kwaves keeps them on the streaming MFMA kernel.  Both
    # meet the contract on a ragged N (65 chunks, the last 8 columns wide).
    N, K = 4104, 1024
    lin = synth.gen_linear(94, N, K)
    pk = packed(lin, N, K)
    x = synth.gen_x(M, K, seed_base=730)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    assert w4.w4a16_plan(M, N, K)["lds"] > 0
    ok, worst = check_contract(_run(x, pk, 0, 0), Y, A)
    assert ok, ("lds", worst)
    for kwaves in (1, 4):
        for splits in (1, 3):
            assert w4.w4a16_plan(M, N, K, splits=splits, kwaves=kwaves)["lds"] == 0
            ok, worst = check_contract(_run(x, pk, kwaves, splits), Y, A)
            assert ok, (kwaves, splits, worst)


@pytest.mark.parametrize("M,kernel", [(1, 1), (5, 0)])
def test_k_splitting_bf16_is_the_rounded_fp32_output(M, kernel):
    N, K = 1000, 1152
    lin = synth.gen_linear(92, N, K)
    pk = packed(lin, N, K)
    x = synth.gen_x(M, K, seed_base=710)
    for kwaves, splits in ((4, 1), (8, 1), (2, 3)):
        y32 = _run(x, pk, kwaves, splits, kernel=kernel)
        yb = _run(x, pk, kwaves, splits, out_bf16=True, kernel=kernel).view(np.uint16)
        assert np.array_equal(yb, round_to_bf16(y32).astype(np.uint16)), (M, kwaves, splits)


def test_decompositions_agree_and_repeat():
    N, K, M = 640, 2816, 5
    lin = synth.gen_linear(93, N, K)
    pk = packed(lin, N, K)
    x = synth.gen_x(M, K, seed_base=720)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    ys = {}
    for kwaves, splits in ((1, 1), (1, 4), (4, 1), (8, 1), (8, 2)):
        a = _run(x, pk, kwaves, splits)
        b = _run(x, pk, kwaves, splits)
        assert np.array_equal(a, b)  # deterministic: fixed summation order
        ys[(kwaves, splits)] = a
    base = ys[(1, 1)]
    for key, y in ys.items():
        # two results, each within the contract of the exact value, differ by at most twice its bound
        assert np.all(np.abs(y.astype(np.float64) - base) <= 8e-3 * A + 1e-30), key
