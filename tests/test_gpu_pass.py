"""GPU parity of the verify pass as one launch (include/w4_pass.h).

The pass is a chain with real data flow, shaped like Llama-3 decoder layers:
q, k and v read the layer input; o reads q's output (standing in for the
attention output, which has q's shape) and waits for q, k and v; gate and up
read o's output; down reads gate's output and waits for gate and up; the next
layer's q, k and v read down's output; the lm_head reads the last down's.
Every linear writes its bf16 output (the next activation) and some also fp32,
scaled by a power-of-two alpha that keeps magnitudes near 1.

The same chain with q|k|v and gate|up fused (o and down reading column
slices of the fused outputs through a row stride) runs in both forms of a
pass: the library chooses per-linear launches for it (one linear per
dependency class), the persistent kernel when asked.

Each output is checked against the oracle applied to the input the linear
actually read (its producer's output buffer after the run), so a consumer
that read its input before the producer finished would not match.  Between
runs the external input changes and every output is filled with NaN first:
a stale or early read shows up as a mismatch or a NaN.  Cases: the
persistent kernel at M = 1 (GEMV) and 2, 5, 8, 16 (MFMA), the per-linear
launches at M = 1, 5, 16 (asked for), 17 and 64, a HIP graph replayed with eager changes between
replays, a forced dependency-wait timeout (spin limit 0) and recovery, a
producer split into K slices across workgroups (the last slice of a chunk
adds the partial tiles) read by its consumer, a consumer reading a column
slice of a fused output through a row stride, and one full-size
Llama-3-70B layer at M = 1 and 5 (its down projection is K-split), separate
and fused (the fused one in both forms).
"""
import math

import numpy as np
import pytest

import synth
from oracle import bf16_bits_to_f64, linear64_gemm, round_to_bf16

from gpu_util import DEV, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

w4 = pytest.importorskip("speculative_decoding_verification_w4a16_amd")


def _alpha(K):
    # a power of two near 1 / (0.02 sqrt(K)): outputs stay near unit scale
    return 2.0 ** -round(math.log2(0.02 * math.sqrt(K)))


class Chain:
    """Weights, buffers and the pass descriptors of a layered chain."""

    def __init__(self, M, H, KV, F, layers, vocab, seed=7000, fp32_leaves=True, fused=False,
                 mode=None):
        self.M = M
        self.lins, self.descs, self.names = [], [], []
        self.x0 = torch.empty((M, H), dtype=torch.int16, device=DEV)
        self.bufs = []
        idx = {}

        def add(name, N, K, x, deps, fp32, ldx=0):
            lin = synth.gen_linear(seed + len(self.lins), N, K)
            pk = w4.repack(to_dev(lin["qweight"]), to_dev(lin["scales"]), to_dev(lin["zeros"]), N, K)
            yb = torch.empty((M, N), dtype=torch.int16, device=DEV)
            y = torch.empty((M, N), dtype=torch.float32, device=DEV) if fp32 else None
            self.bufs += [t for t in (yb, y) if t is not None]
            idx[name] = len(self.lins)
            self.lins.append((lin, pk))
            self.names.append(name)
            self.descs.append(dict(x=x, qweight_t=pk.qweight_t, scales_t=pk.scales_t, zeros_t=pk.zeros_t, y=y,
                                   y_bf16=yb, N=N, K=K, ldx=ldx, alpha=_alpha(K), deps=[idx[d] for d in deps]))
            return yb

        h, hdeps = self.x0, []
        for L in range(layers if fused else 0):
            # q|k|v and gate|up as single linears: o reads the q columns of
            # qkv's output, down the gate columns of gate_up's
            qkv = add(f"qkv{L}", H + 2 * KV, H, h, hdeps, fp32_leaves)
            o = add(f"o{L}", H, H, qkv, [f"qkv{L}"], False, ldx=H + 2 * KV)
            gu = add(f"gate_up{L}", 2 * F, H, o, [f"o{L}"], fp32_leaves)
            h = add(f"down{L}", H, F, gu, [f"gate_up{L}"], True, ldx=2 * F)
            hdeps = [f"down{L}"]
        for L in range(0 if fused else layers):
            q = add(f"q{L}", H, H, h, hdeps, False)
            add(f"k{L}", KV, H, h, hdeps, fp32_leaves)
            add(f"v{L}", KV, H, h, hdeps, fp32_leaves)
            o = add(f"o{L}", H, H, q, [f"q{L}", f"k{L}", f"v{L}"], False)
            g = add(f"gate{L}", F, H, o, [f"o{L}"], False)
            add(f"up{L}", F, H, o, [f"o{L}"], fp32_leaves)
            h = add(f"down{L}", H, F, g, [f"gate{L}", f"up{L}"], True)
            hdeps = [f"down{L}"]
        if vocab:
            add("lm_head", vocab, H, h, hdeps, True)
        self.handle = (w4.w4_pass_create(self.descs, M) if mode is None
                       else w4.w4_pass_create_mode(self.descs, M, mode))

    def close(self):
        w4.w4_pass_destroy(self.handle)

    def set_input(self, seed):
        x = synth.gen_x(self.M, self.x0.shape[1], seed_base=seed)
        self.x0.copy_(to_dev(x))

    def poison(self):
        for t in self.bufs:
            if t.dtype == torch.float32:
                t.fill_(float("nan"))
            else:
                t.fill_(0x7FC0)  # bf16 NaN

    def check(self, what):
        """Every output against the oracle on the input the linear read."""
        torch.cuda.synchronize()
        worst = 0.0
        for (lin, pk), d, name in zip(self.lins, self.descs, self.names):
            x = d["x"].cpu().numpy().view(np.uint16)[:, :d["K"]].copy()  # the columns the linear reads
            assert np.all(np.isfinite(bf16_bits_to_f64(x))), (what, name, "input not finite")
            yb_all = bf16_bits_to_f64(d["y_bf16"].cpu().numpy().view(np.uint16))
            y_all = d["y"].cpu().numpy().astype(np.float64) if d["y"] is not None else None
            al = d["alpha"]
            # column blocks keep the float64 weights of a full-size linear small
            for n0 in range(0, d["N"], 8192):
                n1 = min(d["N"], n0 + 8192)
                Y, A = linear64_gemm(x, lin["qweight"], lin["scales"], lin["zeros"], 128, n0, n1)
                Y, A = Y * al, A * al
                err = np.abs(yb_all[:, n0:n1] - Y)
                bound = 4e-3 * A * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(Y)
                assert np.all(err <= bound), (what, name, n0, float(np.nanmax(err / bound)))
                if y_all is not None:
                    y = y_all[:, n0:n1]
                    assert np.all(np.abs(y - Y) <= 4e-3 * A), (what, name, n0)
                    worst = max(worst, float(np.max(np.abs(y - Y) / np.maximum(4e-3 * A, 1e-300))))
        return worst


SMALL = dict(H=1024, KV=128, F=2816, layers=2, vocab=4096)


AUTO, PERSISTENT, LAUNCHES = w4.W4_PASS_AUTO, w4.W4_PASS_PERSISTENT, w4.W4_PASS_LAUNCHES


@pytest.mark.parametrize("M,mode", [(1, AUTO), (2, AUTO), (5, AUTO), (8, AUTO), (16, AUTO), (17, AUTO), (64, AUTO),
                                    (1, LAUNCHES), (5, LAUNCHES), (16, LAUNCHES)])
def test_chain_against_the_oracle_with_changing_inputs(M, mode):
    # q, k, v share their producers, as do gate and up: 14 linears in 8
    # classes, so the library's choice at M <= 16 is the persistent kernel
    ch = Chain(M, **SMALL, mode=mode)
    info = w4.w4_pass_info(ch.handle)
    assert info["persistent"] == (1 if M <= 16 and mode != LAUNCHES else 0), info
    assert info["units"] == 2 * (16 + 2 + 2 + 16 + 44 + 44 + 16) + 64
    try:
        for run, seed in enumerate((8100, 8200, 8300)):
            ch.set_input(seed)
            ch.poison()
            w4.w4_pass_run(ch.handle)
            w4.w4_pass_check(ch.handle)
            worst = ch.check((M, run))
        print(f"M={M}: {info}, worst err/bound of the fp32 outputs {worst:.2e}")
    finally:
        ch.close()


@pytest.mark.parametrize("M,mode", [(1, AUTO), (5, AUTO), (1, PERSISTENT), (5, PERSISTENT), (16, PERSISTENT),
                                    (33, AUTO)])
def test_fused_chain_in_both_forms(M, mode):
    # q|k|v and gate|up fused: one linear per dependency class, so the
    # library's choice is per-linear launches; the persistent kernel, asked
    # for, computes the same chain (strided reads of the fused outputs)
    ch = Chain(M, **SMALL, fused=True, mode=mode)
    info = w4.w4_pass_info(ch.handle)
    assert info["persistent"] == (1 if mode == PERSISTENT else 0), info
    try:
        for run, seed in enumerate((8150, 8250)):
            ch.set_input(seed)
            ch.poison()
            w4.w4_pass_run(ch.handle)
            w4.w4_pass_check(ch.handle)
            ch.check(("fused", M, mode, run))
    finally:
        ch.close()


@pytest.mark.parametrize("M", [1, 5])
def test_graph_replays_with_eager_changes_between(M):
    ch = Chain(M, **SMALL)
    try:
        ch.set_input(8400)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):  # warm-up outside the capture
            w4.w4_pass_run(ch.handle, s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            w4.w4_pass_run(ch.handle)
        for rep, seed in enumerate((8500, 8600, 8700)):
            ch.set_input(seed)
            ch.poison()
            g.replay()
            w4.w4_pass_check(ch.handle)
            ch.check(("graph", M, rep))
    finally:
        torch.cuda.synchronize()
        ch.close()


def test_forced_wait_timeout_is_reported_and_recovered():
    # spin limit 0: every dependency wait not already satisfied gives up at
    # once (the launch still runs to its end); the check reports it, and the
    # next run with the default limit is correct again
    ch = Chain(1, **SMALL, mode=PERSISTENT)
    try:
        ch.set_input(8800)
        w4.w4_pass_set_spin_limit(ch.handle, 0)
        w4.w4_pass_run(ch.handle)
        with pytest.raises(w4.W4Error) as err:
            w4.w4_pass_check(ch.handle)
        assert err.value.status == w4.W4_ERR_TIMEOUT
        w4.w4_pass_check(ch.handle)  # the flag was cleared
        w4.w4_pass_set_spin_limit(ch.handle, 1 << 24)
        ch.poison()
        w4.w4_pass_run(ch.handle)
        w4.w4_pass_check(ch.handle)
        ch.check("after the timeout")
    finally:
        ch.close()


@pytest.mark.parametrize("M", [1, 5, 16])
def test_k_split_producer_against_the_oracle(M):
    # a producer with few chunks and a long K (8 chunks, 512 groups) is split
    # into K slices across workgroups; the last slice of each chunk adds the
    # partial tiles.  Its consumer reads the summed bf16 output.
    N1, K1, N2 = 512, 65536, 1024
    lin1, lin2 = synth.gen_linear(9100, N1, K1), synth.gen_linear(9101, N2, N1)
    pk1 = w4.repack(to_dev(lin1["qweight"]), to_dev(lin1["scales"]), to_dev(lin1["zeros"]), N1, K1)
    pk2 = w4.repack(to_dev(lin2["qweight"]), to_dev(lin2["scales"]), to_dev(lin2["zeros"]), N2, N1)
    x0 = torch.empty((M, K1), dtype=torch.int16, device=DEV)
    h = torch.empty((M, N1), dtype=torch.int16, device=DEV)
    yf = torch.empty((M, N1), dtype=torch.float32, device=DEV)
    y2 = torch.empty((M, N2), dtype=torch.float32, device=DEV)
    a1 = _alpha(K1)
    descs = [dict(x=x0, qweight_t=pk1.qweight_t, scales_t=pk1.scales_t, zeros_t=pk1.zeros_t, y=yf, y_bf16=h,
                  N=N1, K=K1, alpha=a1, deps=[]),
             dict(x=h, qweight_t=pk2.qweight_t, scales_t=pk2.scales_t, zeros_t=pk2.zeros_t, y=y2, y_bf16=None,
                  N=N2, K=N1, alpha=1.0, deps=[0])]
    hd = w4.w4_pass_create_mode(descs, M, PERSISTENT)
    try:
        info = w4.w4_pass_info(hd)
        assert info["persistent"] == 1 and info["units"] > (N1 // 64) + (N2 // 64), info  # the producer is split
        for seed in (9200, 9300):
            x = synth.gen_x(M, K1, seed_base=seed)
            x0.copy_(to_dev(x))
            for t in (h, yf, y2):
                t.fill_(0x7FC0) if t.dtype == torch.int16 else t.fill_(float("nan"))
            w4.w4_pass_run(hd)
            w4.w4_pass_check(hd)
            torch.cuda.synchronize()
            Y1, A1 = linear64_gemm(x, lin1["qweight"], lin1["scales"], lin1["zeros"], 128, 0, N1)
            y1 = yf.cpu().numpy().astype(np.float64)
            assert np.all(np.abs(y1 - a1 * Y1) <= 4e-3 * a1 * A1), (M, seed, "producer")
            hb = h.cpu().numpy().view(np.uint16)
            assert np.array_equal(hb, round_to_bf16(yf.cpu().numpy()).astype(np.uint16)), (M, seed, "bf16 output")
            Y2, A2 = linear64_gemm(hb, lin2["qweight"], lin2["scales"], lin2["zeros"], 128, 0, N2)
            y2h = y2.cpu().numpy().astype(np.float64)
            assert np.all(np.abs(y2h - Y2) <= 4e-3 * A2), (M, seed, "consumer")
    finally:
        torch.cuda.synchronize()
        w4.w4_pass_destroy(hd)


@pytest.mark.parametrize("M,mode", [(1, PERSISTENT), (5, PERSISTENT), (1, LAUNCHES), (5, LAUNCHES), (17, AUTO),
                                    (64, AUTO)])
def test_consumer_reads_a_column_slice_of_a_fused_output(M, mode):
    # a fused producer (q|k|v-like: N = 1024 + 256 + 256) writes [M, 1536];
    # its consumer reads the first 1024 columns of each row (ldx = 1536), as
    # o reads the q part of a fused q|k|v output -- in the persistent kernel
    # and in per-linear launches
    H, NF, N2 = 1024, 1536, 512
    lin1, lin2 = synth.gen_linear(9400, NF, H), synth.gen_linear(9401, N2, H)
    pk1 = w4.repack(to_dev(lin1["qweight"]), to_dev(lin1["scales"]), to_dev(lin1["zeros"]), NF, H)
    pk2 = w4.repack(to_dev(lin2["qweight"]), to_dev(lin2["scales"]), to_dev(lin2["zeros"]), N2, H)
    x0 = torch.empty((M, H), dtype=torch.int16, device=DEV)
    f = torch.empty((M, NF), dtype=torch.int16, device=DEV)
    y2 = torch.empty((M, N2), dtype=torch.float32, device=DEV)
    descs = [dict(x=x0, qweight_t=pk1.qweight_t, scales_t=pk1.scales_t, zeros_t=pk1.zeros_t, y=None, y_bf16=f,
                  N=NF, K=H, alpha=_alpha(H), deps=[]),
             dict(x=f, qweight_t=pk2.qweight_t, scales_t=pk2.scales_t, zeros_t=pk2.zeros_t, y=y2, y_bf16=None,
                  N=N2, K=H, ldx=NF, alpha=1.0, deps=[0])]
    hd = w4.w4_pass_create_mode(descs, M, mode)
    assert w4.w4_pass_info(hd)["persistent"] == (1 if mode == PERSISTENT else 0)
    try:
        for seed in (9500, 9600):
            x0.copy_(to_dev(synth.gen_x(M, H, seed_base=seed)))
            f.fill_(0x7FC0)
            y2.fill_(float("nan"))
            w4.w4_pass_run(hd)
            w4.w4_pass_check(hd)
            torch.cuda.synchronize()
            xs = f.cpu().numpy().view(np.uint16)[:, :H].copy()  # the slice the consumer reads
            assert np.all(np.isfinite(bf16_bits_to_f64(xs))), (M, seed)
            Y, A = linear64_gemm(xs, lin2["qweight"], lin2["scales"], lin2["zeros"], 128, 0, N2)
            y = y2.cpu().numpy().astype(np.float64)
            assert np.all(np.abs(y - Y) <= 4e-3 * A), (M, seed)
    finally:
        torch.cuda.synchronize()
        w4.w4_pass_destroy(hd)


@pytest.mark.parametrize("M", [1, 5])
def test_full_size_llama_layer(M):
    # one Llama-3-70B decoder layer (hidden 8192, kv 1024, MLP 28672) with the
    # layer's data flow, every column of every output against the oracle
    ch = Chain(M, H=8192, KV=1024, F=28672, layers=1, vocab=0, seed=1000, fp32_leaves=True)
    try:
        ch.set_input(2000)
        ch.poison()
        w4.w4_pass_run(ch.handle)
        w4.w4_pass_check(ch.handle)
        worst = ch.check(("llama layer", M))
        print(f"Llama-3-70B layer M={M}: worst err/bound {worst:.2e}")
    finally:
        ch.close()


@pytest.mark.parametrize("M,mode", [(1, AUTO), (5, AUTO), (5, PERSISTENT)])
def test_full_size_fused_llama_layer(M, mode):
    # one Llama-3-70B decoder layer with q|k|v and gate|up fused (qkv N = 10240,
    # gate_up N = 57344; o and down read column slices of them), in the
    # library's choice of form (per-linear launches) and in the persistent
    # kernel, every column of every output against the oracle
    ch = Chain(M, H=8192, KV=1024, F=28672, layers=1, vocab=0, seed=1100, fp32_leaves=True, fused=True, mode=mode)
    try:
        assert w4.w4_pass_info(ch.handle)["persistent"] == (1 if mode == PERSISTENT else 0)
        ch.set_input(2100)
        ch.poison()
        w4.w4_pass_run(ch.handle)
        w4.w4_pass_check(ch.handle)
        worst = ch.check(("fused llama layer", M, mode))
        print(f"fused Llama-3-70B layer M={M} mode={mode}: worst err/bound {worst:.2e}")
    finally:
        ch.close()


def test_every_m_in_the_persistent_kernel():
    # a producer and its consumer at every M the persistent kernel takes
    # (rows past M repeat row M - 1 in its MFMA form and must never reach an
    # output), against the oracle on the input the consumer read
    N1, K1, N2 = 512, 1024, 256
    lin1, lin2 = synth.gen_linear(9900, N1, K1), synth.gen_linear(9901, N2, N1)
    pk1 = w4.repack(to_dev(lin1["qweight"]), to_dev(lin1["scales"]), to_dev(lin1["zeros"]), N1, K1)
    pk2 = w4.repack(to_dev(lin2["qweight"]), to_dev(lin2["scales"]), to_dev(lin2["zeros"]), N2, N1)
    for M in range(1, 17):
        x = synth.gen_x(M, K1, seed_base=9950)
        x0 = to_dev(x)
        h = torch.full((M, N1), 0x7FC0, dtype=torch.int16, device=DEV)
        y2 = torch.full((M, N2), float("nan"), dtype=torch.float32, device=DEV)
        descs = [dict(x=x0, qweight_t=pk1.qweight_t, scales_t=pk1.scales_t, zeros_t=pk1.zeros_t, y=None, y_bf16=h,
                      N=N1, K=K1, alpha=_alpha(K1), deps=[]),
                 dict(x=h, qweight_t=pk2.qweight_t, scales_t=pk2.scales_t, zeros_t=pk2.zeros_t, y=y2, y_bf16=None,
                      N=N2, K=N1, alpha=1.0, deps=[0])]
        hd = w4.w4_pass_create_mode(descs, M, PERSISTENT)
        try:
            w4.w4_pass_run(hd)
            w4.w4_pass_check(hd)
            torch.cuda.synchronize()
        finally:
            w4.w4_pass_destroy(hd)
        a1 = _alpha(K1)
        Y1, A1 = linear64_gemm(x, lin1["qweight"], lin1["scales"], lin1["zeros"], 128, 0, N1)
        hb = h.cpu().numpy().view(np.uint16)
        err1 = np.abs(bf16_bits_to_f64(hb) - a1 * Y1)
        assert np.all(err1 <= 4e-3 * a1 * A1 * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(a1 * Y1)), (M, "producer")
        Y2, A2 = linear64_gemm(hb, lin2["qweight"], lin2["scales"], lin2["zeros"], 128, 0, N2)
        assert np.all(np.abs(y2.cpu().numpy().astype(np.float64) - Y2) <= 4e-3 * A2), (M, "consumer")



@pytest.mark.parametrize("M", [1, 2, 5, 16])
def test_zero_weight_columns_through_the_persistent_kernel(M):
    # columns of zero weights written with non-zero zero points (q = z = 8, and
    # one column with z = 1..15 per group) give exactly 0 through the pass
    # kernel's own epilogue, fp32 and bf16; a consumer reading that bf16
    # output matches the oracle on what it read
    N, K, g, N2 = 256, 4096, 128, 128
    G = K // g
    rng = np.random.default_rng(1357)
    q = rng.integers(0, 16, size=(K, N))
    z = rng.integers(0, 16, size=(G, N))
    s = (np.float16(2.0 ** -7) * (0.5 + rng.random((G, N)))).astype(np.float16).view(np.uint16)
    zero_cols = [2, 66, 131, 255]
    z[:, zero_cols] = 8
    q[:, zero_cols] = 8
    z[:, 40] = (np.arange(G) % 15) + 1
    q[:, 40] = np.repeat(z[:, 40], g)
    zero_cols.append(40)
    lin = synth.pack_linear(q, z, s)
    lin2 = synth.gen_linear(4242, N2, N)
    pk = w4.repack(to_dev(lin["qweight"]), to_dev(lin["scales"]), to_dev(lin["zeros"]), N, K)
    pk2 = w4.repack(to_dev(lin2["qweight"]), to_dev(lin2["scales"]), to_dev(lin2["zeros"]), N2, N)
    x = synth.gen_x(M, K, seed_base=2468)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    yb = torch.full((M, N), 0x7FC0, dtype=torch.int16, device=DEV)
    y2 = torch.full((M, N2), float("nan"), dtype=torch.float32, device=DEV)
    descs = [dict(x=to_dev(x), qweight_t=pk.qweight_t, scales_t=pk.scales_t, zeros_t=pk.zeros_t, y=y, y_bf16=yb,
                  N=N, K=K, ldx=0, alpha=1.0, deps=[]),
             dict(x=yb, qweight_t=pk2.qweight_t, scales_t=pk2.scales_t, zeros_t=pk2.zeros_t, y=y2, y_bf16=None,
                  N=N2, K=N, ldx=0, alpha=1.0, deps=[0])]
    h = w4.w4_pass_create_mode(descs, M, PERSISTENT)
    try:
        assert w4.w4_pass_info(h)["persistent"] == 1
        w4.w4_pass_run(h)
        w4.w4_pass_check(h)
    finally:
        w4.w4_pass_destroy(h)
    torch.cuda.synchronize()
    y_h = y.cpu().numpy().astype(np.float64)
    yb_h = yb.cpu().numpy().view(np.uint16)
    assert np.all(y_h[:, zero_cols] == 0.0) and np.all((yb_h[:, zero_cols] & 0x7FFF) == 0), M
    Y, A = linear64_gemm(x, lin["qweight"], lin["scales"], lin["zeros"], 128, 0, N)
    assert np.all(A[:, zero_cols] == 0)
    assert np.all(np.abs(y_h - Y) <= 4e-3 * A), M
    Y2, A2 = linear64_gemm(yb_h.copy(), lin2["qweight"], lin2["scales"], lin2["zeros"], 128, 0, N2)
    assert np.all(np.abs(y2.cpu().numpy().astype(np.float64) - Y2) <= 4e-3 * A2), M
