"""Host-side checks of the C ABI: the library loads, exports every symbol the
headers declare, and rejects bad arguments before any HIP call.

Nothing here launches a kernel, so it runs without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h)
           for h in ("w4a16.h", "w4a16_bench.h", "w4_accept.h", "w4_tree_attn.h", "w4_pass.h")]

w4 = pytest.importorskip("speculative_decoding_verification_w4a16_amd")


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(w4\w*)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 12, names
    lib = ctypes.CDLL(w4.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    # and the binding wraps every one of them under the same name
    assert set(names) <= set(w4.exported_symbols())
    for n in names:
        assert callable(getattr(w4, n))


def test_status_strings():
    assert w4.w4_status_str(0) == "W4_OK"
    for s in (1, 2, 3):
        assert w4.w4_status_str(s).startswith("W4_ERR_")
    assert "UNKNOWN" in w4.w4_status_str(99)


def test_repacked_sizes():
    assert w4.w4_repacked_sizes(8192, 8192) == (8192 * 8192 // 2, 8192 * 8192 // 64, 8192 * 8192 // 256)
    # N padded to 64 columns
    assert w4.w4_repacked_sizes(200, 256) == (256 * 256 // 2, 256 * 2 * 2, 256 * 2 // 2)
    for args, code in [((8192, 8192, 64), w4.W4_ERR_UNSUPPORTED), ((8192, 100, 128), w4.W4_ERR_UNSUPPORTED),
                       ((12, 128, 128), w4.W4_ERR_UNSUPPORTED), ((-8, 128, 128), w4.W4_ERR_INVALID)]:
        with pytest.raises(w4.W4Error) as e:
            w4.w4_repacked_sizes(*args)
        assert e.value.status == code


def _lin(x=0x1000, q=0x2000, s=0x3000, z=0x4000, M=4, N=256, K=512, g=128, y=0x100000, kernel=0, splits=0):
    return w4.w4a16_linear_cfg(x, q, s, z, M, N, K, g, y, kernel, splits, stream=0)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), 1), (dict(N=-8), 1), (dict(K=-128), 1),
    (dict(M=65), 2), (dict(g=64), 2), (dict(K=500), 2), (dict(N=12), 2),
    (dict(kernel=1, M=2), 2), (dict(kernel=7), 1), (dict(splits=-1), 1),
    (dict(x=0), 1), (dict(q=0), 1), (dict(s=0), 1), (dict(z=0), 1), (dict(y=0), 1),
    (dict(x=0x1008), 1), (dict(q=0x2004), 1), (dict(s=0x3002), 1), (dict(z=0x4001), 1), (dict(y=0x100002), 1),
    (dict(y=0x1000), 1),            # y overlaps x
    (dict(y=0x2000 + 64), 1),       # y overlaps the weights
])
def test_linear_argument_errors(kw, code):
    with pytest.raises(w4.W4Error) as e:
        _lin(**kw)
    assert e.value.status == code


def test_linear_out_argument_errors():
    def out(**kw):
        a = dict(x=0x1000, q=0x2000, s=0x3000, z=0x4000, M=4, N=256, K=512, g=128, y=0x100000, dt=0)
        a.update(kw)
        return w4.w4a16_linear_out(a["x"], a["q"], a["s"], a["z"], a["M"], a["N"], a["K"], a["g"], a["y"], a["dt"],
                                   stream=0)
    for kw, code in [(dict(dt=2), 1), (dict(dt=-1), 1), (dict(y=0x100008), 1), (dict(y=0x100008, dt=1), 1),
                     (dict(y=0x1000 + 256, dt=1), 1), (dict(M=65, dt=1), 2)]:
        with pytest.raises(w4.W4Error) as e:
            out(**kw)
        assert e.value.status == code, kw
    # a bf16 y of M*N*2 bytes that runs 16 bytes into x overlaps it
    with pytest.raises(w4.W4Error) as e:
        out(y=0x1000 - 4 * 256 * 2 + 16, dt=1)
    assert e.value.status == 1
    assert w4.W4_OUT_F32 == 0 and w4.W4_OUT_BF16 == 1


def test_empty_calls_are_noops():
    # nothing to compute: returns OK without touching memory or the GPU
    _lin(M=0, x=0, q=0, s=0, z=0, y=0)
    _lin(N=0, x=0, q=0, s=0, z=0, y=0)


def test_repack_and_unpack_argument_errors():
    with pytest.raises(w4.W4Error) as e:
        w4.w4_repack(0, 0x3000, 0x4000, 256, 512, 128, 0x10000, 0x20000, 0x30000, stream=0)
    assert e.value.status == 1
    with pytest.raises(w4.W4Error) as e:  # output overlaps input
        w4.w4_repack(0x10000, 0x90000, 0xA0000, 256, 512, 128, 0x10000 + 256, 0xB0000, 0xC0000, stream=0)
    assert e.value.status == 1
    with pytest.raises(w4.W4Error) as e:
        w4.w4_unpack(0x10004, 0x20000, 256, 512, 128, 0x30000, 0x40000, stream=0)
    assert e.value.status == 1
    with pytest.raises(w4.W4Error) as e:
        w4.w4_unpack(0x10000, 0x20000, 256, 512, 96, 0x30000, 0x40000, stream=0)
    assert e.value.status == 2


def test_verify_pass_validates_every_entry_first():
    good = dict(x=0x1000, qweight_t=0x2000, scales_t=0x3000, zeros_t=0x4000, y=0x100000, N=256, K=512)
    bad = dict(good, K=500)
    with pytest.raises(w4.W4Error) as e:
        w4.w4a16_verify_pass([good, bad], M=2, stream=0)
    assert e.value.status == 2
    with pytest.raises(w4.W4Error) as e:
        w4.w4a16_verify_pass([good], M=70, stream=0)
    assert e.value.status == 2


def test_bench_argument_errors():
    with pytest.raises(w4.W4Error):
        w4.w4_bench_read(0x1000, 100, 0x2000, stream=0)
    with pytest.raises(w4.W4Error):
        w4.w4_bench_copy(0x1000, 0x1000 + 16, 64, stream=0)
    assert w4.w4_bench_read_blocks() > 0


@pytest.mark.parametrize("M", [1, 2, 5, 8, 14, 15, 16, 17, 32, 33, 48, 64])
@pytest.mark.parametrize("N,K", [(256, 512), (8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672),
                                 (128256, 8192), (200, 384)])
def test_plans_fit_the_hardware(M, N, K):
    p = w4.w4a16_plan(M, N, K)
    assert p["kernel"] == (w4.W4_KERNEL_GEMV if M == 1 else w4.W4_KERNEL_MFMA)
    assert p["lds"] <= 160 * 1024 - 256  # gfx950 LDS per workgroup, less the static part
    assert 1 <= p["splits"] <= K // 128
    kw = p["kwaves"]
    assert kw in (1, 2, 4, 8) and (M <= 16 or kw == 1)
    chunks = -(-N // 64)
    lds_kernel = M > 16 or (M >= 15 and N >= 4096)  # the LDS-ring kernel
    assert (p["lds"] > 0) == lds_kernel
    if kw == 1:  # four (or, in the LDS kernel, eight) 64-column chunks per workgroup, one per wave
        wv = p["block"] // 64
        assert wv == 4 or (lds_kernel and wv == 8)
        # the LDS kernel may share the row blocks out between 2..4 workgroups
        tiles = -(-chunks // wv) * p["splits"]
        assert p["grid"] % tiles == 0
        rs = p["grid"] // tiles
        mb = -(-M // 16)
        assert rs == 1 or (lds_kernel and rs <= min(4, mb) and tiles * rs <= 256)
        # the narrow k/v projection at M > 16 gets its rows shared out
        if (N, K) == (1024, 8192) and M > 16:
            assert rs == min(mb, 4) if mb != 3 else rs == 3
    else:  # one chunk per workgroup, its kw waves splitting K
        assert p["block"] == 64 * kw and p["grid"] == chunks * p["splits"]
        gps = -(-(K // 128) // p["splits"])
        assert K // 128 - (p["splits"] - 1) * gps >= kw  # every wave has a group
    # the split-K workspace (64 MiB) holds every partial
    assert p["splits"] == 1 or p["splits"] * M * (-(-N // 64) * 64) * 4 <= 64 << 20


def test_random_plans_keep_their_invariants():
    # A seeded sweep over shapes and forced decompositions the model never
    # uses (tiny and ragged N, odd group counts, splits past the group count,
    # every waves-per-chunk choice): every plan fits the hardware, splits K
    # into non-empty runs of whole groups, gives every wave of a K-splitting
    # workgroup a group of its own, covers every chunk, and keeps its partial
    # sums inside the 64 MiB split-K workspace.
    import numpy as np

    rng = np.random.default_rng(2024)
    checked = 0
    for _ in range(4000):
        M = 1 if rng.random() < 0.2 else int(rng.integers(2, 65))  # the GEMV path too
        N = 8 * int(rng.integers(1, 4000 if rng.random() < 0.8 else 20000))
        G = int(rng.integers(1, 300))
        K = 128 * G
        splits = 0 if rng.random() < 0.5 else int(rng.integers(1, G + 8))
        kwaves = int(rng.choice([1, 2, 4, 8])) if M <= 16 and rng.random() < 0.3 else 0
        kernel = w4.W4_KERNEL_MFMA if M == 1 and rng.random() < 0.3 else w4.W4_KERNEL_AUTO
        p = w4.w4a16_plan(M, N, K, kernel=kernel, splits=splits, kwaves=kwaves)
        what = (M, N, K, splits, kwaves, kernel, p)
        chunks, mb = -(-N // 64), -(-M // 16)
        assert p["kernel"] == (w4.W4_KERNEL_GEMV if M == 1 and kernel == w4.W4_KERNEL_AUTO else w4.W4_KERNEL_MFMA), what
        S = p["splits"]
        assert 1 <= S <= G, what
        if splits:
            assert S <= splits, what
        gps = -(-G // S)
        assert -(-G // gps) == S, what  # no split is empty
        assert 0 <= p["lds"] <= 160 * 1024 - 256, what
        lds_kernel = p["lds"] > 0
        assert not lds_kernel or (M > 16 or (M >= 15 and N >= 4096 and kwaves == 0)), what
        kw = p["kwaves"]
        if kwaves:
            assert kw == kwaves or (kw < kwaves and G - (S - 1) * gps < kwaves), what
        if kw > 1:
            assert not lds_kernel and p["block"] == 64 * kw and p["grid"] == chunks * S, what
            assert G - (S - 1) * gps >= kw, what  # every wave of the workgroup has a group
        else:
            wv = p["block"] // 64
            assert wv == 4 or (lds_kernel and wv == 8), what
            tiles = -(-chunks // wv) * S
            assert p["grid"] % tiles == 0, what
            rs = p["grid"] // tiles
            assert rs == 1 or (lds_kernel and 1 < rs <= min(4, mb)), what
        assert 1 <= p["grid"] and p["grid"] * p["block"] < 2 ** 31, what
        assert S == 1 or S * M * chunks * 64 * 4 <= 64 << 20, what
        checked += 1
    assert checked == 4000


def test_forced_plans():
    p = w4.w4a16_plan(1, 8192, 8192, kernel=w4.W4_KERNEL_MFMA, splits=3)
    assert p["kernel"] == w4.W4_KERNEL_MFMA and p["splits"] == 3
    p = w4.w4a16_plan(4, 256, 512, splits=100)
    assert p["splits"] == 4
    p = w4.w4a16_plan(1, 8192, 8192, splits=1, kwaves=8)
    assert (p["kwaves"], p["block"], p["grid"]) == (8, 512, 128)
    p = w4.w4a16_plan(5, 8192, 8192, splits=2, kwaves=2)
    assert (p["kwaves"], p["block"], p["grid"]) == (2, 128, 256)
    p = w4.w4a16_plan(1, 1024, 512, splits=1, kwaves=8)  # 4 groups: at most 4 waves
    assert p["kwaves"] == 4
    p = w4.w4a16_plan(1, 1024, 512, splits=4, kwaves=8)  # 1 group per split
    assert (p["kwaves"], p["block"]) == (1, 256)
    p = w4.w4a16_plan(1, 8192, 8192, splits=1, kwaves=1)
    assert (p["kwaves"], p["block"], p["grid"]) == (1, 256, 32)
    # M = 16 on a wide linear: the LDS kernel, unless the waves are forced
    assert w4.w4a16_plan(16, 8192, 8192)["lds"] > 0
    assert w4.w4a16_plan(16, 8192, 8192, kwaves=1)["lds"] == 0
    for bad, status in ((3, 2), (16, 2), (-1, 1)):
        with pytest.raises(w4.W4Error) as e:
            w4.w4a16_plan(1, 8192, 8192, kwaves=bad)
        assert e.value.status == status
    with pytest.raises(w4.W4Error) as e:
        w4.w4a16_plan(33, 8192, 8192, kwaves=2)  # the M > 16 kernel does not split K in a workgroup
    assert e.value.status == 2


def test_linear_tune_argument_errors():
    # validation happens before any HIP call: fake device addresses never load
    a = 0x10000
    with pytest.raises(w4.W4Error) as e:
        w4.w4a16_linear_tune(a, a + 0x100000, a + 0x200000, a + 0x300000, 1, 256, 512, 128, a + 0x400000,
                             kwaves=-1, stream=0)
    assert e.value.status == 1
    with pytest.raises(w4.W4Error) as e:
        w4.w4a16_linear_tune(a, a + 0x100000, a + 0x200000, a + 0x300000, 1, 256, 512, 128, a + 0x400000,
                             kwaves=5, stream=0)
    assert e.value.status == 2


def test_accept_argument_errors():
    # every check runs before a HIP call: fake device addresses never load
    L, D, U, O, T = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
    V = 128256
    for args, code in [
        (dict(K=-1), 1), (dict(V=-4), 1), (dict(K=65), 2), (dict(V=6), 2), (dict(V=0), 2), (dict(V=(1 << 24) + 4), 2),
        (dict(logits=0), 1), (dict(out=0), 1), (dict(draft=0), 1), (dict(logits=L + 4), 1), (dict(out=O + 2), 1),
        (dict(out=L + 16), 1),  # out inside the logits
    ]:
        a = dict(logits=L, draft=T, K=4, V=V, out=O)
        a.update(args)
        with pytest.raises(w4.W4Error) as e:
            w4.w4_accept_greedy(a["logits"], a["draft"], a["K"], a["V"], a["out"], stream=0)
        assert e.value.status == code, args
    for args, code in [(dict(dl=0), 1), (dict(u=0), 1), (dict(dl=D + 8), 1), (dict(u=U + 2), 1), (dict(out=U), 1)]:
        a = dict(dl=D, u=U, out=O)
        a.update(args)
        with pytest.raises(w4.W4Error) as e:
            w4.w4_accept_sample(L, a["dl"], T, a["u"], 4, V, a["out"], stream=0)
        assert e.value.status == code, args


def test_tree_attention_argument_errors():
    a = dict(q=0x100000, kc=0x200000, vc=0x300000, kd=0x400000, vd=0x500000, m=0x600000, M=5, L=64, H=64, Hkv=8,
             D=128, scale=0.0, out=0x700000)

    def call(**kw):
        b = dict(a)
        b.update(kw)
        return w4.w4_tree_attention(b["q"], b["kc"], b["vc"], b["kd"], b["vd"], b["m"], b["M"], b["L"], b["H"],
                                    b["Hkv"], b["D"], b["scale"], b["out"], stream=0)
    for kw, code in [(dict(M=-1), 1), (dict(L=-1), 1), (dict(D=64), 2), (dict(M=65), 2), (dict(H=60), 2),
                     (dict(q=0), 1), (dict(kc=0), 1), (dict(m=0x600004), 1), (dict(out=0x100000), 1),
                     (dict(q=0x100008), 1), (dict(scale=-1.0), 1), (dict(scale=float("nan")), 1), (dict(Hkv=0), 1)]:
        with pytest.raises(w4.W4Error) as e:
            call(**kw)
        assert e.value.status == code, kw
    assert call(M=0) is None  # nothing to do: no launch, no error
    # the merge choice of the _ex form: anything but AUTO, LAUNCH or LAST is
    # refused (also when there is nothing to do)
    for merge in (-1, 3, 1 << 20):
        with pytest.raises(w4.W4Error) as e:
            w4.w4_tree_attention_ex(a["q"], a["kc"], a["vc"], a["kd"], a["vd"], a["m"], 0, 64, 64, 8, 128, 0.0, merge,
                                    a["out"], stream=0)
        assert e.value.status == w4.W4_ERR_INVALID, merge
    assert w4.w4_tree_attention_ex(a["q"], a["kc"], a["vc"], a["kd"], a["vd"], a["m"], 0, 64, 64, 8, 128, 0.0,
                                   w4.TREE_MERGE_LAST, a["out"], stream=0) is None


def test_tree_attention_plan():
    # Llama-3-70B heads over a 4096-position prefix: the key splits each
    # draft size uses, merged by a second launch by default; either merge can
    # be asked for
    for M, splits in ((1, 33), (5, 22), (64, 8)):
        assert w4.w4_tree_attention_plan(M, 4096, 64, 8) == (splits, w4.TREE_MERGE_LAUNCH), M
        for merge in (w4.TREE_MERGE_LAUNCH, w4.TREE_MERGE_LAST):
            assert w4.w4_tree_attention_plan(M, 4096, 64, 8, merge) == (splits, merge)
    # the default merges in the last workgroup where a tile (at most 16 rows)
    # holds at most 72 KiB of partial rows (130 floats each per split)
    for M, L, Hq, Hkv in ((1, 128, 64, 8), (1, 1024, 64, 8), (1, 2048, 64, 8), (2, 512, 64, 8), (2, 1024, 64, 8),
                          (3, 512, 64, 8), (16, 300, 16, 16), (16, 1000, 16, 16), (1, 100000, 8, 8)):
        splits, used = w4.w4_tree_attention_plan(M, L, Hq, Hkv)
        rows = M * Hq // Hkv
        small = rows <= 16 and splits * rows * 130 * 4 <= 72 << 10
        assert splits > 1 and used == (w4.TREE_MERGE_LAST if small else w4.TREE_MERGE_LAUNCH), (M, L, splits, used)
    assert w4.w4_tree_attention_plan(1, 1024, 64, 8) == (17, w4.TREE_MERGE_LAST)
    assert w4.w4_tree_attention_plan(1, 2048, 64, 8) == (33, w4.TREE_MERGE_LAUNCH)
    assert w4.w4_tree_attention_plan(2, 1024, 64, 8)[1] == w4.TREE_MERGE_LAUNCH
    assert w4.w4_tree_attention_plan(1, 4096, 64, 8)[1] == w4.TREE_MERGE_LAUNCH
    # a single 64-key chunk: one split, nothing to merge
    for merge in (w4.TREE_MERGE_AUTO, w4.TREE_MERGE_LAUNCH, w4.TREE_MERGE_LAST):
        assert w4.w4_tree_attention_plan(3, 20, 64, 8, merge) == (1, w4.TREE_MERGE_AUTO)
    # the extremes of the limits plan (at most 64 splits; every tile has its
    # arrival counter)
    for M, L, Hq, Hkv in ((64, 1 << 20, 256, 1), (64, 1 << 20, 256, 256), (1, 1 << 20, 256, 256),
                          (64, 0, 256, 1), (1, 1, 1, 1), (17, 100000, 64, 8)):
        splits, used = w4.w4_tree_attention_plan(M, L, Hq, Hkv)
        assert 1 <= splits <= 64 and (used != w4.TREE_MERGE_AUTO) == (splits > 1)
    for args, code in (((0, 64, 64, 8), w4.W4_ERR_INVALID), ((65, 64, 64, 8), w4.W4_ERR_UNSUPPORTED),
                       ((1, (1 << 20) + 1, 64, 8), w4.W4_ERR_UNSUPPORTED), ((1, 64, 60, 8), w4.W4_ERR_UNSUPPORTED),
                       ((1, 64, 512, 8), w4.W4_ERR_UNSUPPORTED), ((1, -1, 64, 8), w4.W4_ERR_INVALID)):
        with pytest.raises(w4.W4Error) as e:
            w4.w4_tree_attention_plan(*args)
        assert e.value.status == code, args
    with pytest.raises(w4.W4Error) as e:
        w4.w4_tree_attention_plan(1, 64, 64, 8, 7)
    assert e.value.status == w4.W4_ERR_INVALID


def test_size_limits():
    # the declared limits are accepted (the plan's sizes do not overflow) and
    # one step past either is rejected before any HIP call
    big = 1 << 24
    for M in (1, 5, 17, 64):
        for N, K in ((8, big), (big, 128)):
            p = w4.w4a16_plan(M, N, K)
            assert 1 <= p["splits"] <= K // 128 and p["grid"] >= 1, (M, N, K, p)
            # the split-K workspace (64 MiB) holds every partial
            assert p["splits"] == 1 or p["splits"] * M * (-(-N // 64) * 64) * 4 <= 64 << 20
    for N, K in ((big + 8, 128), (8, big + 128)):
        with pytest.raises(w4.W4Error):
            w4.w4a16_plan(1, N, K)
        rc = w4._c["w4a16_linear"](None, None, None, None, 1, N, K, 128, None, None)
        assert rc == w4.W4_ERR_UNSUPPORTED


def test_noalloc_refuses_a_split_past_its_scratch_before_any_launch():
    # 16 K splits of 64 x 128256 fp32 partials exceed the 64 MiB static
    # scratch: refused on the host (no GPU needed); the same call without a
    # forced split is accepted by validation (it would plan one split)
    with pytest.raises(w4.W4Error) as err:
        w4.w4a16_linear_out_noalloc(0x10000, 0x20000, 0x30000, 0x40000, 64, 128256, 8192, 128, 0x7000000000, 0, 0,
                                    16, stream=0)
    assert err.value.status == w4.W4_ERR_UNSUPPORTED
    with pytest.raises(w4.W4Error) as err:  # misaligned y: rejected like w4a16_linear_out
        w4.w4a16_linear_out_noalloc(0x10000, 0x20000, 0x30000, 0x40000, 4, 256, 512, 128, 0x7000000004, 0, 0, 0,
                                    stream=0)
    assert err.value.status == w4.W4_ERR_INVALID
    assert w4.W4_OK == 0


def _pl(x, y, yb=0, N=256, K=512, deps=(), qt=0x100000, st=0x200000, zt=0x300000, alpha=1.0, ldx=0):
    d = list(deps)
    return w4.W4PassLinear(x, qt, st, zt, y, yb, alpha, N, K, len(d), (ctypes.c_int * 4)(*(d + [0] * 4)[:4]), ldx)


def _create(entries, M=4):
    arr = (w4.W4PassLinear * len(entries))(*entries)
    out = ctypes.c_void_p()
    return w4._c["w4_pass_create"](arr, len(entries), M, 128, ctypes.byref(out))


def test_pass_validation_before_any_hip_call():
    # M = 4, K = 512, N = 256: x is 4 KB, y (fp32) 4 KB; distinct weights per entry
    X0, Y0, Y1 = 0x1000000, 0x2000000, 0x3000000
    wt = lambda i: dict(qt=0x10000000 + i * 0x1000000, st=0x20000000 + i * 0x1000000, zt=0x30000000 + i * 0x1000000)
    ok_chain = [_pl(X0, Y0, **wt(0)), _pl(Y0, Y1, K=256, deps=[0], **wt(1))]
    # a valid chain passes validation and only then needs the device (none here: W4_ERR_HIP)
    rc = _create(ok_chain)
    assert rc in (w4.W4_OK, w4.W4_ERR_HIP), rc
    # a consumer reading the first 512 columns of a 1024-column bf16 output (ldx = 1024)
    strided = [_pl(X0, 0, yb=Y0, N=1024, **wt(0)), _pl(Y0, Y1, K=512, ldx=1024, deps=[0], **wt(1))]
    rc = _create(strided)
    assert rc in (w4.W4_OK, w4.W4_ERR_HIP), rc
    bad = {
        "reads an earlier output without listing it": [_pl(X0, Y0, **wt(0)), _pl(Y0, Y1, K=256, **wt(1))],
        "depends on a later linear": [_pl(X0, Y0, deps=[1], **wt(0)), _pl(X0 + 0x100000, Y1, **wt(1))],
        "depends on itself": [_pl(X0, Y0, deps=[0], **wt(0))],
        "reads the output of a later linear": [_pl(Y1, Y0, **wt(0)), _pl(X0, Y1, **wt(1))],
        "writes its own input": [_pl(X0, X0, **wt(0))],
        "two outputs overlap": [_pl(X0, Y0, **wt(0)), _pl(X0, Y0 + 3968, **wt(1))],
        # a 64-byte bf16 output (4 rows x 8 columns) and an unrelated input in the rest of its line
        "an input shares an output's cache line": [_pl(X0, 0, yb=Y0, N=8, **wt(0)), _pl(Y0 + 64, Y1, **wt(1))],
        "output not 128-byte aligned": [_pl(X0, Y0 + 64, **wt(0))],
        "no output": [_pl(X0, 0, **wt(0))],
        "output over the weights": [_pl(X0, 0x10000000, **wt(0))],
        "zeros not 4-byte aligned": [_pl(X0, Y0, qt=0x10000000, st=0x20000000, zt=0x30000002)],
        "alpha not finite": [_pl(X0, Y0, alpha=float("inf"), **wt(0))],
        "duplicate producer": [_pl(X0, Y0, **wt(0)), _pl(Y0, Y1, K=256, deps=[0, 0], **wt(1))],
        "ldx below K": [_pl(X0, Y0, ldx=256, **wt(0))],
        "ldx not a multiple of 8": [_pl(X0, Y0, ldx=516, **wt(0))],
        # x rows 8 KB apart: the span of 4 rows reaches the later linear's output at X0 + 0x4000
        "a strided input's span meets a later output": [_pl(X0, Y0, ldx=4096, **wt(0)),
                                                        _pl(X0 + 0x200000, X0 + 0x4000, **wt(1))],
        "a strided read of an output not listed": [_pl(X0, 0, yb=Y0, N=1024, **wt(0)),
                                                   _pl(Y0, Y1, K=512, ldx=1024, **wt(1))],
    }
    for name, entries in bad.items():
        assert _create(entries) == w4.W4_ERR_INVALID, name
    # more producers than the limit, group, M, shapes: unsupported
    many = [_pl(X0 + i * 0x10000, Y0 + i * 0x10000, **wt(i)) for i in range(5)]
    many.append(_pl(X0 + 0x900000, Y1, deps=[0, 1, 2, 3, 4], **wt(5)))
    assert _create(many) == w4.W4_ERR_UNSUPPORTED
    assert _create([_pl(X0, Y0, N=4, **wt(0))]) == w4.W4_ERR_UNSUPPORTED
    assert _create([_pl(X0, Y0, **wt(0))], M=65) == w4.W4_ERR_UNSUPPORTED
    out = ctypes.c_void_p()
    arr = (w4.W4PassLinear * 1)(_pl(X0, Y0, **wt(0)))
    assert w4._c["w4_pass_create"](arr, 1, 4, 64, ctypes.byref(out)) == w4.W4_ERR_UNSUPPORTED
    assert w4._c["w4_pass_create"](arr, 1, 4, 128, None) == w4.W4_ERR_INVALID
    # the form: an unknown mode is invalid, the persistent kernel above M = 16
    # unsupported, and both are checked before any HIP call
    for mode in (-1, 3):
        assert w4._c["w4_pass_create_mode"](arr, 1, 4, 128, mode, ctypes.byref(out)) == w4.W4_ERR_INVALID, mode
    assert w4._c["w4_pass_create_mode"](arr, 1, 17, 128, w4.W4_PASS_PERSISTENT,
                                        ctypes.byref(out)) == w4.W4_ERR_UNSUPPORTED
    assert w4._c["w4_pass_create_mode"](arr, 1, 4, 128, w4.W4_PASS_PERSISTENT, None) == w4.W4_ERR_INVALID
    bad_mode = [_pl(X0, Y0, **wt(0)), _pl(Y0, Y1, K=256, **wt(1))]  # an unlisted dependency, any mode
    arr2 = (w4.W4PassLinear * 2)(*bad_mode)
    for mode in (w4.W4_PASS_AUTO, w4.W4_PASS_PERSISTENT, w4.W4_PASS_LAUNCHES):
        assert w4._c["w4_pass_create_mode"](arr2, 2, 4, 128, mode, ctypes.byref(out)) == w4.W4_ERR_INVALID, mode
    assert w4._c["w4_pass_run"](None, None) == w4.W4_ERR_INVALID
    assert w4._c["w4_pass_destroy"](None) == w4.W4_OK


def test_pass_validation_scales_to_large_passes():
    # a chain of 100 000 linears (each reading its predecessor's bf16 output)
    # validates in time that grows like n log n, and one unlisted read at the
    # end of the chain is still found
    import time

    n, M, N, K = 100_000, 4, 256, 256
    X0, OUT, W = 0x10_0000_0000, 0x20_0000_0000, 0x40_0000_0000
    arr = (w4.W4PassLinear * n)()
    for i in range(n):
        wb = W + i * 0x10_0000
        arr[i] = _pl(X0 if i == 0 else OUT + (i - 1) * 4096, 0, yb=OUT + i * 4096, N=N, K=K,
                     deps=() if i == 0 else (i - 1,), qt=wb, st=wb + 0x8_0000, zt=wb + 0xC_0000)
    out = ctypes.c_void_p()
    t0 = time.time()
    rc = w4._c["w4_pass_create"](arr, n, M, 128, ctypes.byref(out))
    took = time.time() - t0
    assert rc in (w4.W4_OK, w4.W4_ERR_HIP), rc
    if rc == w4.W4_OK:
        w4._c["w4_pass_destroy"](out)
    assert took < 10.0, took
    arr[n - 1] = _pl(OUT + (n - 2) * 4096, 0, yb=OUT + (n - 1) * 4096, N=N, K=K,
                     qt=W + (n - 1) * 0x10_0000, st=W + (n - 1) * 0x10_0000 + 0x8_0000,
                     zt=W + (n - 1) * 0x10_0000 + 0xC_0000)
    assert w4._c["w4_pass_create"](arr, n, M, 128, ctypes.byref(out)) == w4.W4_ERR_INVALID



def test_random_tree_plans_keep_their_invariants():
    # seeded sweep over the limits: 1..64 splits, never more than the 64-key
    # chunks, the partial results and arrival counters inside the 48 MiB
    # workspace, and the merge the default picks follows its stated rule
    # (last workgroup only for tiles of at most 16 rows and 72 KiB of partials)
    rng = __import__("numpy").random.default_rng(2024)
    for _ in range(3000):
        M = int(rng.integers(1, 65))
        L = int(rng.choice([0, 1, 63, 64, 65, 500, 4096, 100000, 1 << 20]) if rng.random() < 0.3
                else rng.integers(0, 1 << 17))
        Hkv = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128, 256]))
        Hq = Hkv * int(rng.choice([g for g in (1, 2, 4, 8, 16, 32, 64, 128, 256) if Hkv * g <= 256]))
        splits, used = w4.w4_tree_attention_plan(M, L, Hq, Hkv)
        chunks = -(-(L + M) // 64)
        assert 1 <= splits <= min(64, chunks), (M, L, Hq, Hkv, splits)
        R = M * Hq // Hkv
        rows = 64 if R <= 16 else 128
        tiles = -(-R // rows) * Hkv
        assert tiles * 4 <= 4096, (M, Hq, Hkv)
        if R <= 16 and chunks * tiles <= 288 and 4096 + min(64, chunks) * Hkv * R * 520 <= 48 << 20:
            assert splits == min(64, chunks), (M, L, Hq, Hkv, splits)  # one chunk per split
        if splits > 1:
            assert 4096 + splits * Hkv * R * 130 * 4 <= 48 << 20, (M, L, Hq, Hkv, splits)
            small = R <= 16 and splits * min(R, rows) * 130 * 4 <= 72 << 10
            assert used == (w4.TREE_MERGE_LAST if small else w4.TREE_MERGE_LAUNCH), (M, L, Hq, Hkv, splits, used)
            for m in (w4.TREE_MERGE_LAUNCH, w4.TREE_MERGE_LAST):
                assert w4.w4_tree_attention_plan(M, L, Hq, Hkv, m) == (splits, m)
        else:
            assert used == w4.TREE_MERGE_AUTO
