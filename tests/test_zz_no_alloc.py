"""The allocation-free entry point (w4a16_linear_out_noalloc) against the
allocating one (w4a16_linear_out), through the C ABI.

Both plan every call alike (the static scratch has the workspace's size), so
their outputs must be equal bit for bit, and both within the contract of the
oracle.  Two calls in a row, the second with a smaller input, so the second
reads a scratch that still holds the first call's partials; each on a K split
(the only path that touches the scratch), fp32 and bf16 output, and once with
no split.  A forced split count whose partials exceed the scratch is refused
before any launch.
"""
import numpy as np
import pytest

import synth
from oracle import check_contract, linear64

from gpu_util import DEV, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

w4 = pytest.importorskip("speculative_decoding_verification_w4a16_amd")


def _pk(seed, N, K):
    lin = synth.gen_linear(seed, N, K)
    return lin, w4.repack(to_dev(lin["qweight"]), to_dev(lin["scales"]), to_dev(lin["zeros"]), N, K)


def _both(x, pk, M, out_dtype, splits):
    esz = 2 if out_dtype == w4.W4_OUT_BF16 else 4
    dt = torch.int16 if esz == 2 else torch.float32
    ya = torch.full((M, pk.N), 3, dtype=dt, device=DEV)
    yb = torch.full((M, pk.N), 5, dtype=dt, device=DEV)
    w4.w4a16_linear_out(x, pk.qweight_t, pk.scales_t, pk.zeros_t, M, pk.N, pk.K, 128, ya, out_dtype, 0, splits)
    w4.w4a16_linear_out_noalloc(x, pk.qweight_t, pk.scales_t, pk.zeros_t, M, pk.N, pk.K, 128, yb, out_dtype, 0,
                                splits)
    torch.cuda.synchronize()
    return ya.cpu().numpy(), yb.cpu().numpy()


@pytest.mark.parametrize("out_dtype", [0, 1])
def test_noalloc_equals_the_allocating_entry_point(out_dtype):
    # first call: a wide linear with a 7-way K split at M = 40 (the LDS kernel)
    lin1, pk1 = _pk(501, 3000, 8192)
    x1 = synth.gen_x(40, 8192, seed_base=5100)
    # second call: smaller (fewer rows, columns and groups), 3-way split, M = 5
    lin2, pk2 = _pk(502, 1000, 2048)
    x2 = synth.gen_x(5, 2048, seed_base=5200)
    for lin, pk, x, splits in ((lin1, pk1, x1, 7), (lin2, pk2, x2, 3), (lin2, pk2, x2[:1], 2), (lin2, pk2, x2, 1)):
        M = x.shape[0]
        plan = w4.w4a16_plan(M, pk.N, pk.K, splits=splits)
        assert plan["splits"] == splits, plan
        ya, yb = _both(to_dev(x), pk, M, out_dtype, splits)
        assert np.array_equal(ya, yb), (M, pk.N, splits)
        Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
        if out_dtype == w4.W4_OUT_F32:
            ok, worst = check_contract(yb, Y, A)
            assert ok, (M, worst)
        else:
            yf = (yb.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            assert np.all(np.abs(yf - Y) <= 4e-3 * A * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(Y))


def test_noalloc_automatic_plan_and_refusal():
    lin, pk = _pk(503, 2048, 4096)
    x = synth.gen_x(5, 4096, seed_base=5300)
    ya, yb = _both(to_dev(x), pk, 5, w4.W4_OUT_F32, 0)
    assert np.array_equal(ya, yb)
    # lm_head-sized partials: 16 splits x 64 rows x 128256 columns of fp32 are
    # far past the 64 MiB scratch -- refused, nothing launched
    N, K, M = 128256, 8192, 64
    with pytest.raises(w4.W4Error) as err:
        w4.w4a16_linear_out_noalloc(0x10000, 0x20000, 0x30000, 0x40000, M, N, K, 128, 0x7000000000, 0, 0, 16)
    assert err.value.status == w4.W4_ERR_UNSUPPORTED
