"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

* GP1 unpack: w4_unpack(w4_repack(.)) equals the canonical codes bit for bit;
* layout: the repacked words equal the layout include/w4a16.h documents;
* GP2 one-hot rows: y equals the dequantised weight row exactly;
* GP3 contract: |y - Y64| <= 4e-3 sum|x w| on the tiny linear, ragged shapes
  (N not a multiple of 64, K of 1..9 groups, every m-block boundary) and the
  seven Llama-3-70B-shaped linears at verify sizes M in {1,2,4,5,8,16,32,48,64};
* GP5 row independence; determinism; empty and degenerate calls; the
  verify-pass driver equals separate calls.
"""
import os

import numpy as np
import pytest

import synth
from oracle import linear64, linear64_columns, unpack_qweight, unpack_zeros

from gpu_util import DEV, diagnostics, packed, run_linear, to_dev, torch_mod, unpack_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

w4 = pytest.importorskip("speculative_decoding_verification_w4a16_amd")

FRO_MAX = 1e-5  # fp32 accumulation sits orders of magnitude below the contract


def _layout_words(qweight, N, K):
    """The tile layout as include/w4a16.h documents it (plain loops)."""
    NC, KB = -(-N // 64), K // 32
    q = unpack_qweight(qweight)  # [K, N]
    out = np.zeros((NC, KB, 64, 4), np.uint32)
    for c in range(NC):
        for j in range(4):
            for t in range(16):
                n = 64 * c + 16 * j + t
                if n >= N:
                    continue
                for kb in range(KB):
                    for o in range(4):
                        word = 0
                        for e in range(8):
                            p = e // 2 if e % 2 == 0 else 4 + (e - 1) // 2
                            word |= int(q[32 * kb + 8 * o + e, n]) << (4 * p)
                        out[c, kb, 16 * o + t, j] = ((word << 3) | (word >> 29)) & 0xFFFFFFFF
    return out.reshape(-1)


def test_repack_matches_documented_layout():
    N, K = 200, 256
    lin = synth.gen_linear(31, N, K)
    # groups whose codes all equal their zero point (all weights 0), with
    # zero points 0, 8 and 15, and one group one code short of that
    q, z = unpack_qweight(lin["qweight"]), unpack_zeros(lin["zeros"])
    z[0, 3], z[1, 77], z[0, 199], z[1, 5] = 0, 8, 15, 8
    for g, n in ((0, 3), (1, 77), (0, 199), (1, 5)):
        q[128 * g:128 * (g + 1), n] = z[g, n]
    q[128 + 60, 5] = 7
    lin = synth.pack_linear(q, z, lin["scales"])
    flat = {(0, 3), (1, 77), (0, 199)}
    pk = packed(lin, N, K)
    got = pk.qweight_t.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, _layout_words(lin["qweight"], N, K))
    # scales: (c, G, t, j) -> s[G][64c + 16j + t], 0 for a flat group;
    # zeros nibble j of (c, G, t)
    NC, G = -(-N // 64), K // 128
    st = pk.scales_t.cpu().numpy().view(np.uint16).reshape(NC, G, 16, 4)
    zt = pk.zeros_t.cpu().numpy().view(np.uint16).reshape(NC, G, 16)
    z = unpack_zeros(lin["zeros"])
    for c in range(NC):
        for g in range(G):
            for t in range(16):
                for j in range(4):
                    n = 64 * c + 16 * j + t
                    sv = lin["scales"][g, n] if n < N and (g, n) not in flat else 0
                    zv = z[g, n] if n < N else 0
                    assert st[c, g, t, j] == sv
                    assert (int(zt[c, g, t]) >> (4 * j)) & 15 == zv


@pytest.mark.parametrize("N,K", [(256, 512), (200, 384), (8, 128), (1000, 1152), (64, 128)])
def test_unpack_round_trip_bit_exact(N, K):
    lin = synth.gen_linear(40 + N, N, K)
    q, z = unpack_dev(packed(lin, N, K))
    assert np.array_equal(q, unpack_qweight(lin["qweight"]))
    assert np.array_equal(z, unpack_zeros(lin["zeros"]))


def _check(y, Y, A, what):
    d = diagnostics(y, Y, A)
    assert d["ok"], (what, d)
    assert d["rel_fro"] < FRO_MAX, (what, d)
    return d


@pytest.mark.parametrize("M", [1, 2, 4])
def test_tiny_config_all_kernels_and_splits(M):
    # the tiny linear: K=512, N=256, seed 0, rows 100+i
    N, K = 256, 512
    lin = synth.gen_linear(0, N, K)
    x = synth.gen_x(M, K)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    pk = packed(lin, N, K)
    kernels = [w4.W4_KERNEL_AUTO, w4.W4_KERNEL_MFMA] + ([w4.W4_KERNEL_GEMV] if M == 1 else [])
    for kern in kernels:
        for splits in (0, 1, 2, 3, 4):
            _check(run_linear(x, pk, kern, splits), Y, A, (M, kern, splits))


RAGGED_M = [1, 2, 3, 5, 8, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64]


@pytest.mark.parametrize("N,K", [(320, 1024), (4096, 256)])
def test_every_m_through_the_planner(N, K):
    # every M from 1 to 64 through the planner's kernel choice: the GEMV
    # (M = 1), the streaming MFMA kernel (rows past M repeat row M - 1 and
    # must never reach y), the LDS kernel with one row block (M = 15, 16 on
    # N >= 4096) and with two to four (M = 17..64)
    lin = synth.gen_linear(70 + N, N, K)
    x = synth.gen_x(64, K, seed_base=1700)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    pk = packed(lin, N, K)
    for M in range(1, 65):
        _check(run_linear(x[:M], pk, w4.W4_KERNEL_AUTO, 0), Y[:M], A[:M], (N, K, M))


@pytest.mark.parametrize("N,K", [(200, 384), (8, 128), (1000, 1152), (264, 256)])
def test_ragged_shapes_every_m_block_boundary(N, K):
    lin = synth.gen_linear(50 + N + K, N, K)
    x = synth.gen_x(64, K, seed_base=700)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    pk = packed(lin, N, K)
    for M in RAGGED_M:
        for splits in (0, 1, 2, K // 128):
            _check(run_linear(x[:M], pk, 0, splits), Y[:M], A[:M], (N, K, M, splits))
    # the MFMA kernel also serves M = 1
    _check(run_linear(x[:1], pk, w4.W4_KERNEL_MFMA, 0), Y[:1], A[:1], (N, K, 1, "mfma"))


@pytest.mark.parametrize("M", [1, 5, 40])
def test_every_split_reduction_width(M):
    # The split-K reduction launch loads up to 2, 4, 8, 16 or 32 partials in
    # one batch and loops over batches of 32 beyond that: force split counts
    # in every width and past it (K = 64 groups, so each count below splits
    # the groups exactly) for each streaming kernel.
    N, K = 200, 8192
    lin = synth.gen_linear(81, N, K)
    x = synth.gen_x(M, K, seed_base=900)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    pk = packed(lin, N, K)
    for splits in (2, 3, 4, 5, 8, 13, 16, 22, 32, 64):
        plan = w4.w4a16_plan(M, N, K, splits=splits)
        assert plan["splits"] == splits, plan
        _check(run_linear(x, pk, 0, splits), Y, A, (M, splits))


@pytest.mark.parametrize("M,kernel", [(1, 1), (1, 2), (16, 0), (40, 0), (64, 0)])
def test_one_hot_rows_bit_exact(M, kernel):
    # GP2: x = e_k for every k of the K = 512 linear (all nibble positions,
    # group edges, the first and last k), M rows per call through each
    # kernel path, unsplit and split three ways: y equals the dequantised
    # weight row (q - z) * s exactly
    N, K = 136, 512
    lin = synth.gen_linear(60, N, K)
    pk = packed(lin, N, K)
    x = synth.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    Y, _ = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    for i0 in range(0, K, M):
        rows = slice(i0, min(K, i0 + M))
        for splits in (1, 3):
            y = run_linear(x[rows], pk, kernel, splits)
            assert np.array_equal(y.astype(np.float64), Y[rows]), (i0, splits)


def test_empty_and_degenerate_calls():
    N, K = 256, 512
    lin = synth.gen_linear(70, N, K)
    pk = packed(lin, N, K)
    y = torch.full((4, N), 7.0, device=DEV)
    x = to_dev(synth.gen_x(4, K))
    w4.w4a16_linear(x, pk.qweight_t, pk.scales_t, pk.zeros_t, 0, N, K, 128, y)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)  # M = 0 writes nothing
    w4.w4a16_linear(x, pk.qweight_t, pk.scales_t, pk.zeros_t, 4, N, 0, 128, y)
    torch.cuda.synchronize()
    assert torch.all(y == 0.0)  # K = 0: empty sum


def test_determinism_and_row_independence():
    N, K = 1024, 2048
    lin = synth.gen_linear(80, N, K)
    pk = packed(lin, N, K)
    x = synth.gen_x(64, K, seed_base=900)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    for M in (5, 64):
        y1 = run_linear(x[:M], pk)
        y2 = run_linear(x[:M], pk)
        assert np.array_equal(y1, y2)
        _check(y1, Y[:M], A[:M], M)
        # GP5: each row against its own single-token pass
        worst = 0.0
        for i in range(M):
            yi = run_linear(x[i:i + 1], pk)
            err = np.abs(yi[0].astype(np.float64) - y1[i])
            worst = max(worst, float((err / (2 * 4e-3 * np.maximum(A[i], 1e-300))).max()))
        assert worst <= 1.0


@pytest.mark.parametrize("M", [1, 5, 16, 40, 64])
def test_verify_pass_against_the_oracle(M):
    # every kernel path in one pass: the GEMV (M = 1), the streaming MFMA
    # kernel, the one-row-block LDS kernel (M = 16 on the 4096-column linear),
    # row slices (M > 16 on the narrow ones) and the full LDS kernel; every
    # output against the oracle, and bit for bit against separate calls
    shapes = [(256, 512), (1024, 512), (512, 1024), (4096, 512)]
    if M == 16:
        assert w4.w4a16_plan(M, 4096, 512)["lds"] > 0 and w4.w4a16_plan(M, 1024, 512)["lds"] == 0
    lins, descs, ys = [], [], []
    xs, xh = {}, {}
    for i, (N, K) in enumerate(shapes):
        lin = synth.gen_linear(90 + i, N, K)
        pk = packed(lin, N, K)
        if K not in xs:
            xh[K] = synth.gen_x(M, K, seed_base=950 + K)
            xs[K] = to_dev(xh[K])
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        lins.append((lin, pk, K))
        descs.append(dict(x=xs[K], qweight_t=pk.qweight_t, scales_t=pk.scales_t, zeros_t=pk.zeros_t, y=y, N=N, K=K))
        ys.append(y)
    w4.w4a16_verify_pass(descs, M)
    torch.cuda.synchronize()
    for (lin, pk, K), y in zip(lins, ys):
        Y, A = linear64(xh[K], lin["qweight"], lin["scales"], lin["zeros"])
        _check(y.cpu().numpy(), Y, A, ("verify pass", M, pk.N, K))
        ref = w4.linear(xs[K], pk)
        torch.cuda.synchronize()
        assert torch.equal(ref, y)


# ---------------------------------------------------------------------------
# Llama-3-70B-shaped linears (plain decode, sequence and tree drafts)
# ---------------------------------------------------------------------------

def test_eight_chunk_workgroups_ragged():
    # Wide linears at M >= 15 run eight chunks per workgroup.  N here leaves
    # the last workgroup half empty (436 chunks, 4 past a multiple of 8) and
    # its last chunk partly padded; M = 15 and 16 (one row block: each line
    # of the activation copy is written by two waves), 17, 40 (three row
    # blocks: the copy duplicates a line) and 64 (four); sampled columns
    # include the first, a middle and the last chunk; the planner's split
    # count and a forced odd one both run eight-chunk workgroups.
    N, K = 27896, 8192
    lin = synth.gen_linear(83, N, K)
    pk = packed(lin, N, K)
    x = synth.gen_x(64, K, seed_base=950)
    slices = [(0, 64), (13824, 13888), (N - 120, N)]
    refs = [linear64_columns(x, lin["qweight"], lin["scales"], lin["zeros"], 128, a, b) for a, b in slices]
    for M in (15, 16, 17, 40, 64):
        for splits in (0, 3):
            plan = w4.w4a16_plan(M, N, K, splits=splits)
            assert plan["block"] == 512 and plan["lds"] > 0, plan
            y = run_linear(x[:M], pk, 0, splits)
            for (a, b), (Y, A) in zip(slices, refs):
                _check(y[:, a:b], Y[:M], A[:M], (M, splits, a))


def test_one_row_block_lds_kernel_ragged():
    # M = 15 and 16 on a linear of 4096 or more columns run the LDS kernel
    # with one row block, here four chunks per workgroup: 128 chunks, the
    # last 8 columns short; every column checked, with the planner's split
    # count, none, and three splits of 16 groups (a short last split).
    N, K = 8136, 2048
    lin = synth.gen_linear(87, N, K)
    pk = packed(lin, N, K)
    x = synth.gen_x(16, K, seed_base=960)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    for M in (15, 16):
        for splits in (0, 1, 3):
            plan = w4.w4a16_plan(M, N, K, splits=splits)
            assert plan["block"] == 256 and plan["lds"] > 0, plan
            _check(run_linear(x[:M], pk, 0, splits), Y[:M], A[:M], (M, splits))
    # M = 14 stays on the streaming kernel
    assert w4.w4a16_plan(14, N, K)["lds"] == 0
    _check(run_linear(x[:14], pk), Y[:14], A[:14], (14, 0))


def test_row_slices_ragged():
    # Narrow linears at M > 16 share their row blocks out between two to four
    # workgroups per column tile and split (row slices of one or two blocks;
    # the last slice short or a single row).  16 chunks, the last 24 columns
    # short; every column checked at every slice boundary, with the
    # planner's split count, none, an odd forced count, and 20 requested
    # (16 run), which leaves room for two slices of two blocks at M > 32.
    N, K = 1000, 8192
    lin = synth.gen_linear(89, N, K)
    pk = packed(lin, N, K)
    x = synth.gen_x(64, K, seed_base=970)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    chunks = -(-N // 64)
    for M in (17, 31, 32, 33, 47, 48, 49, 63, 64):
        for splits in (0, 1, 5, 20):
            plan = w4.w4a16_plan(M, N, K, splits=splits)
            rs = plan["grid"] // (-(-chunks // (plan["block"] // 64)) * plan["splits"])
            assert rs > 1 and plan["lds"] > 0, plan
            if splits == 20 and M > 32:
                assert rs == 2 and plan["lds"] == 24960, plan  # two row blocks per workgroup
            _check(run_linear(x[:M], pk, 0, splits), Y[:M], A[:M], (M, splits, rs))


def test_lm_head_full_size_sampled_columns():
    # The widest linear of the sweep at full size (N = 128256 = 2004 chunks, so
    # the last eight-chunk workgroup is half empty), its seed as in the sweep,
    # through every kernel path the planner picks for M = 1 .. 64; columns
    # sampled at the start, the middle and the end.
    N, K = synth.LM_HEAD[1], synth.LM_HEAD[2]
    lin = synth.gen_linear(20000, N, K)
    pk = packed(lin, N, K)
    x = synth.gen_x(64, K)
    slices = [(0, 64), (64128, 64192), (N - 64, N)]
    refs = [linear64_columns(x, lin["qweight"], lin["scales"], lin["zeros"], 128, a, b) for a, b in slices]
    del lin
    for M in (1, 5, 14, 16, 17, 40, 64):
        y = run_linear(x[:M], pk)
        for (a, b), (Y, A) in zip(slices, refs):
            _check(y[:, a:b], Y[:M], A[:M], ("lm_head", M, a))


def test_largest_k_one_chunk():
    # K at the library's limit (2**24, 131072 groups) on one padded chunk: the
    # planner splits K 194 or 512 ways (the reduction loops over batches of
    # partials), and row offsets into x reach 16 * 2**24 elements.
    N, K = 8, 1 << 24
    lin = synth.gen_linear(85, N, K)
    pk = packed(lin, N, K)
    x = synth.gen_x(17, K, seed_base=990)
    Y, A = linear64(x, lin["qweight"], lin["scales"], lin["zeros"])
    del lin
    for M in (1, 5, 17):
        _check(run_linear(x[:M], pk), Y[:M], A[:M], ("K=2**24", M))


# plain decode, sequence drafts, and tree drafts at every row-block count
# (17, 33, 49 open a row block; on k and v they start two, three and four
# row slices)
VERIFY_M = [1, 2, 4, 5, 8, 15, 16, 17, 32, 33, 48, 49, 63, 64]


@pytest.fixture(scope="module")
def layer():
    out = {}
    for idx, (name, N, K) in enumerate(synth.LAYER_LINEARS):
        lin = synth.gen_linear(1000 + idx, N, K)
        out[name] = (lin, packed(lin, N, K), N, K)
    return out


@pytest.mark.parametrize("name", [n for n, _, _ in synth.LAYER_LINEARS])
def test_layer_linear_unpack_bit_exact(layer, name):
    lin, pk, N, K = layer[name]
    q, z = unpack_dev(pk)
    assert np.array_equal(q, unpack_qweight(lin["qweight"]))
    assert np.array_equal(z, unpack_zeros(lin["zeros"]))


@pytest.mark.parametrize("name", [n for n, _, _ in synth.LAYER_LINEARS])
def test_layer_linear_contract_sampled_columns(layer, name):
    lin, pk, N, K = layer[name]
    x = synth.gen_x(64, K)
    rng = np.random.default_rng(1234)
    mid = int(rng.integers(1, N // 64 - 1)) * 64
    slices = [(0, 64), (mid, mid + 64), (N - 64, N)]
    refs = [linear64_columns(x, lin["qweight"], lin["scales"], lin["zeros"], 128, a, b) for a, b in slices]
    for M in VERIFY_M:
        y = run_linear(x[:M], pk)
        for (a, b), (Y, A) in zip(slices, refs):
            _check(y[:, a:b], Y[:M], A[:M], (name, M, a))
