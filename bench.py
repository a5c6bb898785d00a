#!/usr/bin/env python3
"""Verify-pass benchmark of the W4A16 linear on one MI355X.

Workload (the full-model verify sweep): a Llama-3-70B-shaped target with 80
decoder layers of seven int4 linears (q 8192->8192, k/v 8192->1024,
o 8192->8192, gate/up 8192->28672, down 28672->8192) and an int4 lm_head
8192->128256, uint4 codes with fp16 scales and uint4 zeros per group of 128,
W ~ N(0, 0.02) quantised round-to-nearest; layer L's linear idx uses seed
10000 + 7L + idx and the lm_head seed 20000.  ~36.1 GB of packed weights stay
resident in HBM.  One *step* is three verify passes, at M = 1 (plain decode),
M = 5 (a sequence draft) and M = 64 (a flattened tree draft).

A pass keeps the model's data dependencies, with the projections that share
an input fused (the layer's weights concatenated): layer L's qkv (q|k|v,
N = 10240) reads the layer input (layer L-1's down output; layer 0: a seeded
input), o reads the q columns of qkv's output (standing in for the attention
output, which has q's shape), gate_up (gate|up, N = 57344) reads o's output,
down reads the gate columns of gate_up's output, and the lm_head reads the
last down output: 321 linears.  Every linear writes its result as bf16 (the
next layer's activation type), scaled by a power of two (1/2 for K = 8192,
1/4 for K = 28672) that keeps the activations near unit scale over 80
layers.  A pass is one pass object (include/w4_pass.h) in the form the
library chooses -- for this pass, one linear per dependency class,
per-linear launches at every M -- captured once in a HIP graph and
replayed.  Algorithmic bytes per linear: 0.51953125 N K (codes, scales,
zeros) + 2 M K (x) + 2 M N (the bf16 output).

Printed JSON line: `value` is the step's effective HBM throughput (algorithmic
bytes of the three passes / step time, TB/s); per-M microseconds per pass,
t(M)/t(1), roofline fractions; for comparison the same pass in the
persistent-kernel form (M = 1, 5), the unfused pass (561 linears, in the
library's choice of form: the persistent kernel at M = 1 and 5) and the 561
linears as independent launches (no dependencies, fp32 outputs); the
measured HBM read ceiling, the oracle's host throughput on a bounded sample
and the oracle checks (every output column of three seeded-random layers and
a 512-column slice of the lm_head, against the oracle on the inputs each
linear read) ride along.

Usage: python bench.py [--gpus 1] [--steps 10] [--warmup 3]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import queue
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16, published
PASS_M = (1, 5, 64)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(M: int, N: int, K: int, out_bytes: int = 4) -> int:
    """Algorithmic HBM bytes of one linear: packed codes (N K / 2), fp16 scales
    and uint4 zeros per group of 128 (N K / 64 + N K / 256), x once (2 M K)
    and y once (out_bytes M N: 4 for fp32, 2 for bf16)."""
    return N * K // 2 + N * K // 64 + N * K // 256 + 2 * M * K + out_bytes * M * N


def alg_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the oracle on the host")
    p.add_argument("--no-parity", action="store_true", help="skip the oracle spot checks")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the fused-projection and acceptance measurements (profiling runs of the sweep)")
    p.add_argument("--pass-mode", choices=("auto", "persistent", "launches"), default="auto",
                   help="the form of the measured passes at M <= 16 (default: the library's choice)")
    p.add_argument("--headline-only", action="store_true",
                   help="only the measured passes (profiling runs): no comparison passes, extras, parity or CPU "
                        "baseline")
    p.add_argument("--shapes", action="store_true",
                   help="per-linear report instead of the sweep: each decoder shape and the lm_head at every M of "
                        "--m, graph-replayed over rotating weight copies (>= --rotate-gib) so HBM, not the 256 MB "
                        "MALL, serves them; one JSON line per (shape, M)")
    p.add_argument("--floor", action="store_true",
                   help="instead of the sweep: plain streaming reads of each linear's packed bytes (one launch "
                        "each), an empty launch, and their sum over a pass")
    p.add_argument("--tree", action="store_true",
                   help="instead of the sweep: only the tree-draft verify attention measurement (one JSON line)")
    p.add_argument("--tree-merge-sweep", action="store_true",
                   help="instead of the sweep: tree attention with each merge of the key splits forced, over "
                        "prefix lengths and draft sizes (one JSON line per case)")
    p.add_argument("--m", default="1,2,4,5,8,16,32,48,64", help="M grid for --shapes")
    p.add_argument("--names", default="q,k,v,o,gate,up,down,lm_head", help="linears for --shapes")
    p.add_argument("--splits", type=int, default=0, help="force the K split count in --shapes (0 = planner)")
    p.add_argument("--kernel", choices=("auto", "gemv", "mfma"), default="auto",
                   help="force the kernel in --shapes (auto = planner; gemv only at M = 1)")
    p.add_argument("--kwaves", type=int, default=0,
                   help="force the waves splitting a chunk's K range in --shapes (0 = planner; M <= 16)")
    p.add_argument("--rotate-gib", type=float, default=2.0)
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="instead of running: turn two rocprofv3 --pmc runs of the sweep (FETCH_SIZE, WRITE_SIZE; "
                        "taken with --copy-calib) into profiles/traffic.json")
    p.add_argument("--curve-from", metavar="SHAPES_JSONL",
                   help="instead of running: the markdown tables of a --shapes run's JSON lines (us per call, "
                        "t(M)/t(1) with one layer's sum, TB/s, roofline fraction)")
    p.add_argument("--trace-summary", metavar="TRACE_DIR",
                   help="instead of running: per-linear kernel time of each measured pass from a rocprofv3 "
                        "--kernel-trace run of --headline-only (run_kernel_trace.csv)")
    p.add_argument("--copy-calib", type=int, default=0,
                   help="with --shapes: also run w4_bench_copy over this many MiB (HBM counter calibration)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# model construction: host generation (threads) -> pinned -> HBM -> repack
# ---------------------------------------------------------------------------

def model_specs():
    import synth

    specs = []
    for L in range(synth.N_LAYERS):
        for idx, (name, N, K) in enumerate(synth.LAYER_LINEARS):
            specs.append(dict(layer=L, name=name, N=N, K=K, seed=10000 + 7 * L + idx))
    name, N, K = synth.LM_HEAD
    specs.append(dict(layer=None, name=name, N=N, K=K, seed=20000))
    return specs


class PinnedSlot:
    """A pinned host buffer big enough for the largest linear's canonical arrays."""

    def __init__(self, torch, max_nk: int, max_groups_n: int):
        self.q = torch.empty(max_nk // 8, dtype=torch.int32, pin_memory=True)
        self.s = torch.empty(max_groups_n, dtype=torch.int16, pin_memory=True)
        self.z = torch.empty(max_groups_n // 8, dtype=torch.int32, pin_memory=True)

    def views(self, N, K):
        G = K // 128
        return {"qweight": self.q[: N * K // 8].numpy().reshape(K // 8, N),
                "scales": self.s[: G * N].numpy().view(np.uint16).reshape(G, N),
                "zeros": self.z[: G * N // 8].numpy().reshape(G, N // 8)}

    def tensors(self, N, K):
        G = K // 128
        return self.q[: N * K // 8], self.s[: G * N], self.z[: G * N // 8]


def build_model(torch, w4, keep_layers, keep_linears=()):
    """Generate, upload and repack every linear.  Returns (packed, host_copies)
    where host_copies holds the canonical arrays of the layers the oracle
    checks and of `keep_linears`."""
    import synth

    dev = torch.device("cuda:0")
    specs = model_specs()
    max_nk = max(s["N"] * s["K"] for s in specs)
    max_gn = max(s["N"] * s["K"] // 128 for s in specs)
    slots = [PinnedSlot(torch, max_nk, max_gn) for _ in range(3)]
    free = queue.Queue()
    for s in slots:
        free.put(s)
    ready = queue.Queue(maxsize=len(slots))
    threads = synth._threads()

    def producer():
        for spec in specs:
            slot = free.get()
            synth.gen_linear(spec["seed"], spec["N"], spec["K"], out=slot.views(spec["N"], spec["K"]), nthreads=threads)
            ready.put((spec, slot))

    th = threading.Thread(target=producer, daemon=True)
    th.start()
    stage_q = torch.empty(max_nk // 8, dtype=torch.int32, device=dev)
    stage_s = torch.empty(max_gn, dtype=torch.int16, device=dev)
    stage_z = torch.empty(max_gn // 8, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    packed = {}
    host = {}
    t0 = time.time()
    for i in range(len(specs)):
        spec, slot = ready.get()
        N, K = spec["N"], spec["K"]
        key = (spec["layer"], spec["name"])
        if spec["layer"] in keep_layers or key in keep_linears:
            host[key] = {k: v.copy() for k, v in slot.views(N, K).items()}
        hq, hs, hz = slot.tensors(N, K)
        dq, ds, dz = stage_q[: hq.numel()], stage_s[: hs.numel()], stage_z[: hz.numel()]
        dq.copy_(hq, non_blocking=True)
        ds.copy_(hs, non_blocking=True)
        dz.copy_(hz, non_blocking=True)
        G = K // 128
        pk = w4.repack(dq.view(K // 8, N), ds.view(G, N), dz.view(G, N // 8), N, K)
        ev = torch.cuda.Event()
        ev.record(stream)
        ev.synchronize()  # the slot's host data has been consumed
        free.put(slot)
        packed[key] = pk
        if (i + 1) % 70 == 0 or i + 1 == len(specs):
            log(f"[bench] model: {i + 1}/{len(specs)} linears resident ({time.time() - t0:.1f} s)")
    th.join()
    del stage_q, stage_s, stage_z
    torch.cuda.synchronize()
    return packed, host


# ---------------------------------------------------------------------------
# measurement pieces
# ---------------------------------------------------------------------------

def hbm_read_ceiling(torch, w4, nbytes=8 << 30, reps=5):
    """Achievable HBM read bandwidth: one 128-bit-load pass over 8 GiB."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    buf.fill_(1)
    sink = torch.empty(w4.w4_bench_read_blocks(), dtype=torch.int32, device="cuda:0")
    w4.w4_bench_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        w4.w4_bench_read(buf, nbytes, sink)
        e.record()
        e.synchronize()
        best = max(best, nbytes / (s.elapsed_time(e) * 1e-3) / 1e9)
    del buf
    return best


def source_digest():
    """Digest of the sources that define the verify-linear kernels (what the
    HBM byte counters in profiles/traffic.json were taken on)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "speculative_decoding_verification_w4a16_amd", "csrc")
    for f in ("w4_internal.h", "w4_device.h", "w4a16_kernels.hip", "w4_pass.hip"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(M: int):
    """HBM bytes per launch of the pass at M (the whole pass for the
    persistent pass kernel, one linear for per-linear launches) from the
    committed PMC summary, if it was taken on the current kernel sources;
    else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("source_digest") != source_digest():
        return None
    ent = data.get("passes", {}).get(str(M))
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def cpu_baseline(host, budget_s=20.0):
    """The oracle, as it stands, on a bounded sample of the workload: the
    sweep's linears held in host memory (layer 0, then the parity layers), each
    at the pass M = 1, 5 and 64, one (layer, M, linear) unit at a time until
    about budget_s seconds of CPU work.  Besides the rate: the host's core
    count, the BLAS numpy calls and the threads it used, the oracle's two
    steps timed apart per (linear, M) -- dequantisation (unpack, (q - z) * s
    in float64) and the float64 products -- and one unit on a single thread."""
    import synth
    from oracle import linear64
    from oracle.w4a16_ref import _rows as rows64, _weights64 as weights64
    from threadpoolctl import threadpool_info, threadpool_limits

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    blas = [dict(api=i.get("user_api"), lib=i.get("internal_api"), version=i.get("version"),
                 threads=i.get("num_threads")) for i in threadpool_info() if i.get("user_api") == "blas"]
    blas_threads = max([b["threads"] or 0 for b in blas] or [cores])
    units, secs, nbytes = 0, 0.0, 0
    steps = {}  # "linear M" -> [dequant s, product s, units]
    layers = sorted({L for (L, _) in host if L is not None})
    xs = {}
    for L in layers:
        for M in PASS_M:
            for name, N, K in synth.LAYER_LINEARS:
                key = (L, name)
                if key not in host or secs > budget_s:
                    continue
                lin = host[key]
                if K not in xs:
                    xs[K] = synth.gen_x(64, K)
                # linear64 is its two steps in turn: the float64 weights
                # (unpack, dequantise), then the products row by row
                t0 = time.perf_counter()
                W64 = weights64(lin["qweight"], lin["scales"], lin["zeros"], 128)
                t1 = time.perf_counter()
                rows64(xs[K][:M], W64)
                t2 = time.perf_counter()
                del W64
                secs += t2 - t0
                nbytes += alg_bytes(M, N, K)
                units += 1
                st = steps.setdefault(f"{name} M={M}", [0.0, 0.0, 0])
                st[0] += t1 - t0
                st[1] += t2 - t1
                st[2] += 1
    # one unit on one thread: layer 0's q at M = 1
    single = None
    key = (layers[0], "q") if layers else None
    if key in host:
        lin = host[key]
        N, K = next((n, k) for (nm, n, k) in synth.LAYER_LINEARS if nm == "q")
        with threadpool_limits(limits=1, user_api="blas"):
            t = time.perf_counter()
            linear64(synth.gen_x(1, K), lin["qweight"], lin["scales"], lin["zeros"])
            dt = time.perf_counter() - t
        single = {"linear": f"q {N}x{K}", "M": 1, "seconds": round(dt, 3),
                  "value": round(alg_bytes(1, N, K) / dt / 1e12, 6), "unit": "TB/s", "threads": 1}
    return {"value": round(nbytes / secs / 1e12, 6), "unit": "TB/s", "cores": blas_threads, "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "affinity_cores": cores, "blas": blas,
            "steps_seconds": {k: {"dequant": round(v[0], 3), "product": round(v[1], 3), "units": v[2]}
                              for k, v in steps.items()},
            "single_thread": single,
            "sample": f"float64 oracle (numpy, BLAS threads={blas_threads}) on {units} (layer, M, linear) units of "
                      f"the sweep (layers {layers}, M in {list(PASS_M)}, in that order until ~{budget_s:.0f} s): "
                      f"{nbytes / 1e9:.3f} GB of algorithmic traffic in {secs:.2f} s; steps_seconds: the "
                      f"oracle's two steps (float64 weights, then products) timed apart"}


# ---------------------------------------------------------------------------
# the verify pass with the model's data dependencies (one pass object per M)
# ---------------------------------------------------------------------------

def layer_alpha(K: int) -> float:
    """Power-of-two output scale near 1 / (0.02 sqrt(K)): 1/2 at K = 8192, 1/4
    at K = 28672, so activations stay near unit scale through 80 layers."""
    import math

    return 2.0 ** -round(math.log2(0.02 * math.sqrt(K)))


def dependent_pass(torch, w4, packed, M, input_seed=2000):
    """The pass object of the sweep at M: every linear reads the bf16 output
    of its producer (see the module docstring) and writes its own bf16
    output to a buffer of its own.  Returns (handle, outputs by (layer,
    name), layer-0 input tensor, the descriptors)."""
    import synth

    dev = "cuda:0"
    H = synth.LAYER_LINEARS[0][2]
    h0 = torch.from_numpy(synth.gen_x(M, H, seed_base=input_seed).view(np.int16)).to(dev)
    outs, descs, index = {}, [], {}
    h, hdeps = h0, []

    def add(L, name, x, deps):
        pk = packed[(L, name)]
        y = torch.empty((M, pk.N), dtype=torch.int16, device=dev)
        outs[(L, name)] = y
        index[(L, name)] = len(descs)
        descs.append(dict(x=x, qweight_t=pk.qweight_t, scales_t=pk.scales_t, zeros_t=pk.zeros_t, y=None,
                          y_bf16=y, N=pk.N, K=pk.K, alpha=layer_alpha(pk.K), deps=[index[d] for d in deps],
                          key=(L, name)))
        return y

    for L in range(synth.N_LAYERS):
        q = add(L, "q", h, hdeps)
        add(L, "k", h, hdeps)
        add(L, "v", h, hdeps)
        o = add(L, "o", q, [(L, "q"), (L, "k"), (L, "v")])
        g = add(L, "gate", o, [(L, "o")])
        add(L, "up", o, [(L, "o")])
        h = add(L, "down", g, [(L, "gate"), (L, "up")])
        hdeps = [(L, "down")]
    add(None, "lm_head", h, hdeps)
    handle = w4.w4_pass_create(descs, M)
    return handle, outs, h0, descs


def fused_dependent_pass(torch, w4, fpk, M, input_seed=2000, mode=None):
    """The dependent pass over the fused projections: per layer qkv (N =
    10240) reads the layer input; o reads the q part of qkv's output (its
    first 8192 columns, ldx = 10240); gate_up (N = 57344) reads o's output;
    down reads the gate part of gate_up's output (its first 28672 columns,
    ldx = 57344); the lm_head reads the last down's output.  Returns (handle,
    outputs by (layer, name), layer-0 input tensor, the descriptors)."""
    import synth

    dev = "cuda:0"
    H = synth.LAYER_LINEARS[0][2]
    h0 = torch.from_numpy(synth.gen_x(M, H, seed_base=input_seed).view(np.int16)).to(dev)
    outs, descs, index = {}, [], {}
    h, hdeps = h0, []

    def add(L, name, x, deps, K, ldx=0):
        pk = fpk[(L, name)]
        y = torch.empty((M, pk.N), dtype=torch.int16, device=dev)
        outs[(L, name)] = y
        index[(L, name)] = len(descs)
        descs.append(dict(x=x, qweight_t=pk.qweight_t, scales_t=pk.scales_t, zeros_t=pk.zeros_t, y=None,
                          y_bf16=y, N=pk.N, K=K, ldx=ldx, alpha=layer_alpha(K), deps=[index[d] for d in deps],
                          key=(L, name)))
        return y

    F = synth.LAYER_LINEARS[4][1]
    for L in range(synth.N_LAYERS):
        qkv = add(L, "qkv", h, hdeps, H)
        o = add(L, "o", qkv, [(L, "qkv")], H, ldx=qkv.shape[1])
        gu = add(L, "gate_up", o, [(L, "o")], H)
        h = add(L, "down", gu, [(L, "gate_up")], F, ldx=gu.shape[1])
        hdeps = [(L, "down")]
    add(None, "lm_head", h, hdeps, H)
    handle = w4.w4_pass_create(descs, M) if mode is None else w4.w4_pass_create_mode(descs, M, mode)
    return handle, outs, h0, descs


def fused_dependent_parity(w4, host, descs, check_layers, n0):
    """Every output column of the checked layers' fused linears (each part
    against its own linear's oracle on the input the linear read) and the
    lm_head slice; the same bound as dependent_pass_parity."""
    import synth
    from oracle import bf16_bits_to_f64, linear64_gemm

    parts = {"qkv": ("q", "k", "v"), "o": ("o",), "gate_up": ("gate", "up"), "down": ("down",),
             "lm_head": ("lm_head",)}
    worst = 0.0
    for d in descs:
        L, name = d["key"]
        if L not in check_layers and name != "lm_head":
            continue
        x = d["x"].cpu().numpy().view(np.uint16)[:, :d["K"]].copy()  # the columns the linear read
        y = bf16_bits_to_f64(d["y_bf16"].cpu().numpy().view(np.uint16))
        c0 = 0
        for part in parts[name]:
            lin = host[(None if part == "lm_head" else L, part)]
            N = lin["scales"].shape[1]
            cols = [(n0, n0 + 512)] if part == "lm_head" else [(a, min(N, a + 4096)) for a in range(0, N, 4096)]
            for a, b in cols:
                Y, A = linear64_gemm(x, lin["qweight"], lin["scales"], lin["zeros"], 128, a, b)
                Y, A = Y * d["alpha"], A * d["alpha"]
                bound = 4e-3 * A * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(Y)
                r = float(np.max(np.abs(y[:, c0 + a:c0 + b] - Y) / bound))
                if not r <= 1.0:
                    raise AssertionError(f"fused parity failure: layer {L} {name}/{part} cols {a}:{b} ratio {r}")
                worst = max(worst, r)
            c0 += N
    return worst


def dependent_pass_parity(torch, w4, host, descs, check_layers, n0, M):
    """Every output column of the checked layers' linears, and columns
    [n0, n0 + 512) of the lm_head, against the oracle applied to the input
    buffer each linear read (its producer's bf16 output after the pass):
    |y - alpha Y64| <= 4e-3 alpha A64 (1 + 2^-8) + 2^-8 |alpha Y64| (the
    contract plus the bf16 rounding of the output).  Returns the worst ratio."""
    from oracle import bf16_bits_to_f64, linear64_gemm

    torch.cuda.synchronize()
    worst = 0.0
    for d in descs:
        L, name = d["key"]
        if L not in check_layers and name != "lm_head":
            continue
        lin = host[(L, name)]
        x = d["x"].cpu().numpy().view(np.uint16)
        y = bf16_bits_to_f64(d["y_bf16"].cpu().numpy().view(np.uint16))
        cols = [(n0, n0 + 512)] if name == "lm_head" else [(a, min(d["N"], a + 4096)) for a in range(0, d["N"], 4096)]
        for a, b in cols:
            Y, A = linear64_gemm(x, lin["qweight"], lin["scales"], lin["zeros"], 128, a, b)
            Y, A = Y * d["alpha"], A * d["alpha"]
            bound = 4e-3 * A * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(Y)
            r = float(np.max(np.abs(y[:, a:b] - Y) / bound))
            if not r <= 1.0:
                raise AssertionError(f"parity failure: layer {L} {name} M={M} cols {a}:{b} ratio {r}")
            worst = max(worst, r)
    return worst


# ---------------------------------------------------------------------------

FUSED_GROUPS = [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")), ("down", ("down",))]


def fuse_projections(w4, packed):
    """The sweep's packed weights with the projections that share an input
    concatenated on the device (the tile layout is chunk-major): per layer qkv
    (N = 10240), o, gate_up (N = 57344), down; and the lm_head."""
    import synth

    fpk = {}
    for L in range(synth.N_LAYERS):
        for fname, names in FUSED_GROUPS:
            fpk[(L, fname)] = (packed[(L, names[0])] if len(names) == 1
                               else w4.concat_packed([packed[(L, n)] for n in names]))
    fpk[(None, "lm_head")] = packed[(None, "lm_head")]
    return fpk


def fused_sweep(torch, w4, fpk, xs, host, check_layers, args):
    """The same pass with the projections that share an input fused: per
    layer qkv (N = 10240) | o | gate+up (N = 57344) | down, plus the lm_head
    (321 launches instead of 561), with fp32 output and with the bf16
    epilogue, as independent launches (no data flow between them).
    Graph-replayed like the sweep; parity of the fused linears on the checked
    layers' sampled columns (fp32 output against the contract, bf16 output
    against the rounded fp32 output)."""
    import synth
    from oracle import check_contract, linear64_columns

    dev = "cuda:0"
    groups = FUSED_GROUPS
    fspec = []
    for L in range(synth.N_LAYERS):
        for fname, names in groups:
            pk = fpk[(L, fname)]
            fspec.append((L, fname, pk.N, pk.K))
    fspec.append((None, "lm_head", synth.LM_HEAD[1], synth.LM_HEAD[2]))
    yf = {N: torch.empty((64, N), dtype=torch.float32, device=dev) for N in {s[2] for s in fspec}}
    yb = {N: torch.empty((64, N), dtype=torch.int16, device=dev) for N in {s[2] for s in fspec}}
    out = {"launches_per_pass": len(fspec), "us_per_pass": {}, "us_per_pass_bf16_out": {}, "tbps_per_pass": {},
           "roofline_frac_per_pass": {}}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            fn()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        reps = max(3, args.steps)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(reps):
            g.replay()
        s1.record()
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) * 1e3 / reps

    for M in PASS_M:
        descs = [dict(x=xs[K][:M], qweight_t=fpk[(L, f)].qweight_t, scales_t=fpk[(L, f)].scales_t,
                      zeros_t=fpk[(L, f)].zeros_t, y=yf[N][:M], N=N, K=K) for (L, f, N, K) in fspec]
        us = timed(lambda: w4.w4a16_verify_pass(descs, M))

        def bf16_pass():
            for (L, f, N, K) in fspec:
                w4.linear(xs[K][:M], fpk[(L, f)], y=yb[N][:M], out_bf16=True)

        us_b = timed(bf16_pass)
        B = sum(alg_bytes(M, N, K) for (_, _, N, K) in fspec)
        F = sum(alg_flops(M, N, K) for (_, _, N, K) in fspec)
        t_roof = max(B / (HBM_PEAK_GBS * 1e9), F / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6
        out["us_per_pass"][str(M)] = round(us, 1)
        out["us_per_pass_bf16_out"][str(M)] = round(us_b, 1)
        out["tbps_per_pass"][str(M)] = round(B / (us * 1e-6) / 1e12, 4)
        out["roofline_frac_per_pass"][str(M)] = round(t_roof / us, 4)

    if args.no_parity:
        out["worst_err_over_bound"] = None
    else:
        rng = np.random.default_rng(5)
        worst = 0.0
        for M in PASS_M:
            for L in check_layers:
                for fname, names in groups:
                    if len(names) == 1:
                        continue
                    pk = fpk[(L, fname)]
                    K = pk.K
                    y = w4.linear(xs[K][:M], pk).cpu().numpy()
                    ybits = w4.linear(xs[K][:M], pk, out_bf16=True).cpu().numpy().view(np.uint16)
                    if not np.array_equal(ybits, oracle_round_bf16(y)):
                        raise SystemExit(f"fused bf16 output != rounded fp32 output: layer {L} {fname} M={M}")
                    c0 = 0
                    for n in names:
                        lin = host[(L, n)]
                        N = lin["scales"].shape[1]
                        a = int(rng.integers(0, N // 64)) * 64
                        Y, A = linear64_columns(synth.gen_x(M, K), lin["qweight"], lin["scales"], lin["zeros"], 128,
                                                a, a + 64)
                        ok, w = check_contract(y[:, c0 + a:c0 + a + 64], Y, A)
                        if not ok:
                            raise SystemExit(f"fused parity failure: layer {L} {fname}/{n} M={M} ratio {w}")
                        worst = max(worst, w)
                        c0 += N
        out["worst_err_over_bound"] = worst
    del yf, yb
    torch.cuda.empty_cache()
    return out


def acceptance_bench(torch, w4, args):
    """The acceptance step on the lm_head's logits (vocabulary 128256) for a
    sequence draft (K = 4, the M = 5 pass) and a 63-token chain (the M = 64
    pass), greedy and sampled: microseconds per call (graph-replayed, 50 calls
    per replay), the bytes it must read -- target rows (K+1)*V*4, draft rows
    K*V*4 and the final row's target and draft logits again (sampled) -- and
    the rate against the 8 TB/s roofline.  Synthetic logits: target N(0, 2),
    draft = target + N(0, 0.7); drafted tokens drawn from the draft; uniforms
    drawn until every decision clears its boundary; (accepted, next) checked
    against the oracle."""
    from oracle import accept_greedy, accept_sampled, decision_margins, softmax64

    dev = "cuda:0"
    V = 128256  # the lm_head's vocabulary
    rng = np.random.default_rng(17)
    out = {}
    for K in (4, 63):
        L = rng.normal(0.0, 2.0, (K + 1, V)).astype(np.float32)
        Q = (L[:K] + rng.normal(0.0, 0.7, (K, V))).astype(np.float32)
        q = softmax64(Q)
        d = np.array([rng.choice(V, p=q[j]) for j in range(K)], np.int32)
        for _ in range(200):
            u = rng.random(K + 1).astype(np.float32)
            m = decision_margins(L, Q, d, u.astype(np.float64))
            if min(m[:-1]) > 1e-5 and m[-1] > 2e-6:
                break
        Ld, Qd = torch.from_numpy(L).to(dev), torch.from_numpy(Q).to(dev)
        dd, ud = torch.from_numpy(d).to(dev), torch.from_numpy(u).to(dev)
        res = torch.empty(2, dtype=torch.int32, device=dev)
        ok = True
        for mode in ("greedy", "sampled"):
            def call():
                if mode == "greedy":
                    w4.w4_accept_greedy(Ld, dd, K, V, res)
                else:
                    w4.w4_accept_sample(Ld, Qd, dd, ud, K, V, res)
            call()
            torch.cuda.synchronize()
            got = tuple(int(v) for v in res.cpu())
            exp = accept_greedy(L, d) if mode == "greedy" else accept_sampled(L, Q, d, u.astype(np.float64))
            ok = ok and got == exp
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=torch.cuda.Stream()):
                for _ in range(50):
                    call()
            g.replay()
            torch.cuda.synchronize()
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(3, args.steps)
            s0.record()
            for _ in range(reps):
                g.replay()
            s1.record()
            torch.cuda.synchronize()
            us = s0.elapsed_time(s1) * 1e3 / (reps * 50)
            nbytes = (K + 1) * V * 4 + (K * V * 4 + 2 * V * 4 if mode == "sampled" else 0)
            out[f"K{K}_{mode}"] = {"us_per_call": round(us, 2), "bytes": nbytes,
                                   "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                                   "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                   "oracle_match": got == exp}
            del g
        out[f"K{K}_accepted_sampled"] = int(exp[0])
    return out


def tree_attention_bench(torch, w4, args):
    """Tree-draft verify attention of one layer (64 query heads over 8
    key/value heads, head dim 128) over a 4096-position KV prefix, for the
    pass M = 1, a 5-token chain (sequence draft) and a 64-token random tree
    (tree draft): microseconds per call (graph-replayed, 20 calls per replay;
    with the default merge of the key splits, and with each merge forced),
    the KV bytes it must read, the flops it must do (q.k and p.v over every
    visible key), and the rates against the 8 TB/s and 2.5 PFLOP/s rooflines.
    Synthetic bf16 inputs N(0, 1); outputs checked against the oracle."""
    from oracle import ancestor_masks, attention_weight_mass, tree_attention

    dev = "cuda:0"
    Hq, Hkv, D, L = 64, 8, 128, 4096
    rng = np.random.default_rng(23)

    def bf16(shape):
        u = rng.normal(0.0, 1.0, shape).astype(np.float32).view(np.uint32).astype(np.uint64)
        b = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        return b, (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    out = {"L": L, "heads": [Hq, Hkv, D]}
    kcb, kc = bf16((L, Hkv, D))
    vcb, vc = bf16((L, Hkv, D))
    td = lambda b: torch.from_numpy(b.view(np.int16)).to(dev)
    kcd, vcd = td(kcb), td(vcb)
    for name, M, parents in (("M1", 1, [-1]), ("M5_chain", 5, list(range(-1, 4))),
                             ("M64_tree", 64, [-1] + [int(rng.integers(-1, i)) for i in range(1, 64)])):
        qb, q = bf16((M, Hq, D))
        kdb, kd = bf16((M, Hkv, D))
        vdb, vd = bf16((M, Hkv, D))
        masks = ancestor_masks(parents)
        qd, kdd, vdd = td(qb), td(kdb), td(vdb)
        md = torch.from_numpy(masks.view(np.int64)).to(dev)
        o = torch.empty((M, Hq, D), dtype=torch.float32, device=dev)
        args_o = (q, kc, vc, kd, vd, masks)
        ref, mass = tree_attention(*args_o), attention_weight_mass(*args_o)

        def timed(merge):
            w4.tree_attention(qd, kcd, vcd, kdd, vdd, md, out=o, merge=merge)
            torch.cuda.synchronize()
            worst = float(np.max(np.abs(o.cpu().numpy() - ref) / (1e-2 * mass + 1e-6)))
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=torch.cuda.Stream()):
                for _ in range(20):
                    w4.tree_attention(qd, kcd, vcd, kdd, vdd, md, out=o, merge=merge)
            g.replay()
            torch.cuda.synchronize()
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(3, args.steps)
            s0.record()
            for _ in range(reps):
                g.replay()
            s1.record()
            torch.cuda.synchronize()
            del g
            return s0.elapsed_time(s1) * 1e3 / (reps * 20), worst

        by_merge = {name_m: timed(m) for name_m, m in (("launch", w4.TREE_MERGE_LAUNCH), ("last", w4.TREE_MERGE_LAST))}
        us, worst = timed(w4.TREE_MERGE_AUTO)
        splits, used = w4.w4_tree_attention_plan(M, L, Hq, Hkv)
        visible = sum(bin(int(m)).count("1") for m in masks)
        nbytes = 2 * L * Hkv * D * 2 + 2 * M * Hkv * D * 2 + M * Hq * D * 2 + M * Hq * D * 4
        flops = 4.0 * Hq * D * (M * L + visible)
        out[name] = {"M": M, "us_per_call": round(us, 2), "bytes": nbytes, "flops": flops,
                     "TBps": round(nbytes / (us * 1e-6) / 1e12, 3), "TFLOPs": round(flops / (us * 1e-6) / 1e12, 2),
                     "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "frac_mfma": round(flops / (us * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
                     "worst_err_over_bound": round(max([worst] + [w for _, w in by_merge.values()]), 5),
                     "splits": splits, "merge": {0: "none", 1: "launch", 2: "last"}[used],
                     "us_by_merge": {k: round(t, 2) for k, (t, _) in by_merge.items()}}
    return out


def tree_merge_sweep(torch, w4):
    """Microseconds per tree attention call (64 query heads over 8 key/value
    heads; chain drafts; N(0, 1) bf16 inputs; graph-replayed, 20 calls per
    replay, best of 3 x 10 replays) with the key splits merged by a second
    launch and by the last workgroup of each tile, for M = 1..64 over
    prefixes of 128..8192 positions; the merge the default takes; and the
    largest difference between the two outputs."""
    dev = "cuda:0"
    Hq, Hkv, D = 64, 8, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    bf = lambda *shape: torch.randn(*shape, device=dev, generator=gen).to(torch.bfloat16)
    for L in (128, 256, 512, 1024, 2048, 4096, 8192):
        kc, vc = bf(L, Hkv, D), bf(L, Hkv, D)
        for M in (1, 2, 5, 8, 16, 64):
            q, kd, vd = bf(M, Hq, D), bf(M, Hkv, D), bf(M, Hkv, D)
            masks = torch.tensor([((1 << (i + 1)) - 1) - (1 << 64 if i == 63 else 0) for i in range(M)],
                                 dtype=torch.int64, device=dev)
            o = torch.empty(M, Hq, D, device=dev)
            splits, used = w4.w4_tree_attention_plan(M, L, Hq, Hkv)
            row = {"M": M, "L": L, "splits": splits, "default": {0: "none", 1: "launch", 2: "last"}[used]}
            outs = {}
            for name, merge in (("launch", w4.TREE_MERGE_LAUNCH), ("last", w4.TREE_MERGE_LAST)):
                w4.tree_attention(q, kc, vc, kd, vd, masks, out=o, merge=merge)
                torch.cuda.synchronize()
                outs[name] = o.clone()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=torch.cuda.Stream()):
                    for _ in range(20):
                        w4.tree_attention(q, kc, vc, kd, vd, masks, out=o, merge=merge)
                g.replay()
                torch.cuda.synchronize()
                best = float("inf")
                for _ in range(3):
                    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    s0.record()
                    for _ in range(10):
                        g.replay()
                    s1.record()
                    torch.cuda.synchronize()
                    best = min(best, s0.elapsed_time(s1) * 1e3 / 200)
                row[name + "_us"] = round(best, 2)
                del g
            row["max_abs_diff"] = float((outs["launch"] - outs["last"]).abs().max())
            print(json.dumps(row), flush=True)


def oracle_round_bf16(y):
    from oracle import round_to_bf16

    return round_to_bf16(y)


def cost_table(us_per_pass):
    """Speed-up of speculative decoding over plain decoding from the measured
    pass times (the verification-cost model of the package's cost_model)."""
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "cost_model", os.path.join(ROOT, "speculative_decoding_verification_w4a16_amd", "cost_model.py"))
    cm = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(cm)
    return cm.table(us_per_pass)


def copy_calibration(torch, w4, mib):
    """A plain copy of known size (mib MiB read and written, five times): what
    the HBM byte counters read for it scales their readings of the kernels."""
    nb = mib << 20
    src = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    src.fill_(3)
    for _ in range(5):
        w4.w4_bench_copy(dst, src, nb)
    torch.cuda.synchronize()
    del src, dst


def traffic_from_pmc(fetch_dir, write_dir, copy_mib, out_path):
    """HBM bytes per launch of each sweep pass from two rocprofv3 --pmc runs
    of the sweep (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch; taken with
    --headline-only so that only the measured passes run), each scaled by
    what the counter reads for w4_bench_copy of copy_mib MiB.  A launch is
    one dispatch of the persistent pass kernel (the whole pass; GEMV form at
    M = 1, MFMA form at M = 5) or one linear (its kernel plus the split-K
    reduction dispatched right after it when K is split).  Writes
    profiles/traffic.json (tagged with the kernel-source digest) and returns
    it."""
    import csv
    import glob

    def per_dispatch(d, counter):
        vals, names = {}, {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                i = int(r["Dispatch_Id"])
                vals[i] = vals.get(i, 0.0) + float(r["Counter_Value"])
                names[i] = r["Kernel_Name"]
        return vals, names

    def pass_of(name):
        # (M, what a launch is): the persistent pass kernel is a whole pass,
        # the per-linear kernels one linear each
        for key, m, kind in (("w4_pass_kernel<0", "1", "pass"), ("w4_pass_kernel<1", "5", "pass"),
                             ("w4a16_gemv_kernel", "1", "linear"), ("w4a16_mfma_direct_kernel", "5", "linear"),
                             ("w4a16_mfma_lds_kernel", "64", "linear")):
            if key in name:
                return m, kind
        return None, None

    out = {"source_digest": source_digest(), "copy_calibration_mib": copy_mib, "launch": {}, "passes": {}}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals, names = per_dispatch(d, counter)
        copies = [vals[i] for i in vals if "bench_copy" in names[i]]
        factor = (copy_mib * 1024.0) / (sum(copies) / len(copies))  # true KiB per counted KiB
        out[counter + "_factor"] = round(factor, 4)
        sums, counts, cur = {}, {}, None
        for i in sorted(vals):
            n = names[i]
            if "splitk_reduce" in n:
                if cur is not None:  # the reduction of the linear launched just before
                    sums[cur] += vals[i] * factor * 1024
                continue
            cur, kind = pass_of(n)
            if cur is not None:
                out["launch"][cur] = kind
                sums[cur] = sums.get(cur, 0.0) + vals[i] * factor * 1024
                counts[cur] = counts.get(cur, 0) + 1
        for m in sums:
            ent = out["passes"].setdefault(m, {"launches_counted": counts[m]})
            ent[counter.lower() + "_bytes_per_launch"] = int(sums[m] / counts[m])
    for m, ent in out["passes"].items():
        ent["hbm_bytes_per_launch"] = ent.get("fetch_size_bytes_per_launch", 0) + \
            ent.get("write_size_bytes_per_launch", 0)
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def curve_tables(path):
    """Markdown tables of a --shapes run (its JSON lines in `path`): us per
    call, t(M)/t(1) (with one decoder layer summed, separate and fused),
    effective TB/s and the roofline fraction, per linear and M."""
    d = {}
    for line in open(path):
        if line.startswith("{"):
            r = json.loads(line)
            if "linear" in r and "M" in r:
                d[(r["linear"], r["M"])] = r
    names = [n for n in ("q", "k", "v", "o", "gate", "up", "down", "lm_head", "qkv", "gate_up")
             if any(k[0] == n for k in d)]
    ms = sorted({k[1] for k in d})
    head = "| linear | " + " | ".join(f"M = {m}" for m in ms) + " |\n|---|" + "---|" * len(ms)
    layers = [("one layer, 7 launches", ("q", "k", "v", "o", "gate", "up", "down")),
              ("one layer, fused (4 launches)", ("qkv", "o", "gate_up", "down"))]
    out = []

    def table(title, value, fmt, sums=False):
        out.append(f"## {title}\n\n{head}")
        for n in names:
            out.append(f"| {n} | " + " | ".join(fmt % value(n, m) for m in ms) + " |")
        for label, parts in (layers if sums else ()):
            if all((p_, m) in d for p_ in parts for m in ms):
                t1 = sum(d[(p_, ms[0])]["us"] for p_ in parts)
                out.append(f"| {label} | " + " | ".join("%.2f" % (sum(d[(p_, m)]["us"] for p_ in parts) / t1)
                                                        for m in ms) + " |")
        out.append("")

    table("us per call (median)", lambda n, m: d[(n, m)]["us"], "%.1f")
    table("t(M) / t(1)", lambda n, m: d[(n, m)]["us"] / d[(n, ms[0])]["us"], "%.2f", sums=True)
    table("Effective TB/s (algorithmic bytes / t)", lambda n, m: d[(n, m)]["tbps"], "%.2f")
    table("Fraction of the roofline, max(bytes / 8 TB/s, flops / 2.5 PFLOP/s) / t",
          lambda n, m: d[(n, m)]["roofline_frac"], "%.2f")
    table("Spread: (max - min) / median of the repeats",
          lambda n, m: (d[(n, m)]["us_max"] - d[(n, m)]["us_min"]) / d[(n, m)]["us"], "%.3f")
    return "\n".join(out)


def trace_summary(trace_dir):
    """Per-linear kernel time of the measured passes from a rocprofv3
    --kernel-trace run of `bench.py --headline-only`: every dispatch of a
    per-linear kernel, plus the split-K reduction dispatched right after it,
    is one linear of the pass at the M that kernel serves (as in
    traffic_from_pmc); a persistent pass kernel dispatch is a whole pass.
    Returns {M: {kernel, linears (dispatches), mean_us (kernel + its
    reduction), kernel_mean_us (kernel alone)}}."""
    import csv
    import glob

    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    keys = (("w4_pass_kernel<0", "1"), ("w4_pass_kernel<1", "5"), ("w4a16_gemv_kernel", "1"),
            ("w4a16_mfma_direct_kernel", "5"), ("w4a16_mfma_lds_kernel", "64"))
    out, cur = {}, None
    for r in rows:
        name = r["Kernel_Name"]
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if "splitk_reduce" in name:
            if cur is not None:
                out[cur]["total_us"] += dur
            continue
        cur = next((m for k, m in keys if k in name), None)
        if cur is None:
            continue
        e = out.setdefault(cur, {"kernels": set(), "linears": 0, "total_us": 0.0, "kernel_us": 0.0})
        short = name.replace("(anonymous namespace)::", "").replace("void ", "")
        e["kernels"].add(short[:short.index(">(") + 1] if ">(" in short else short.split("(")[0])
        e["linears"] += 1
        e["total_us"] += dur
        e["kernel_us"] += dur
    return {m: {"kernels": sorted(e["kernels"]), "dispatches": e["linears"],
                "mean_us": round(e["total_us"] / e["linears"], 3),
                "kernel_mean_us": round(e["kernel_us"] / e["linears"], 3)} for m, e in sorted(out.items())}


def shapes_report(args):
    """Per-linear microseconds and effective TB/s (the tiny, plain-decode,
    sequence-draft and tree-draft configurations' shapes)."""
    import torch

    import speculative_decoding_verification_w4a16_amd as w4
    import synth

    dev = "cuda:0"
    w4.w4_init()
    table = {name: (N, K, 1000 + i) for i, (name, N, K) in enumerate(synth.LAYER_LINEARS)}
    table["lm_head"] = (synth.LM_HEAD[1], synth.LM_HEAD[2], 20000)
    table["qkv"] = (10240, 8192, 21000)      # the fused projections' shapes
    table["gate_up"] = (57344, 8192, 22000)
    Ms = [int(v) for v in args.m.split(",")]
    if args.copy_calib:
        copy_calibration(torch, w4, args.copy_calib)
    for name in args.names.split(","):
        N, K, seed = table[name]
        lin = synth.gen_linear(seed, N, K)
        base = w4.repack(torch.from_numpy(lin["qweight"]).to(dev), torch.from_numpy(lin["scales"].view(np.int16)).to(dev),
                         torch.from_numpy(lin["zeros"]).to(dev), N, K)
        R = max(2, int(args.rotate_gib * (1 << 30) // base.nbytes))
        copies = [base] + [w4.PackedLinear(base.qweight_t.clone(), base.scales_t.clone(), base.zeros_t.clone(), N, K)
                           for _ in range(R - 1)]
        x = torch.from_numpy(synth.gen_x(max(Ms), K).view(np.int16)).to(dev)
        y = torch.empty((max(Ms), N), dtype=torch.float32, device=dev)
        kern = {"auto": w4.W4_KERNEL_AUTO, "gemv": w4.W4_KERNEL_GEMV, "mfma": w4.W4_KERNEL_MFMA}[args.kernel]
        for M in Ms:
            plan = w4.w4a16_plan(M, N, K, kernel=kern, splits=args.splits, kwaves=args.kwaves)
            for pk in copies[:2]:
                w4.linear(x[:M], pk, y=y[:M], kernel=kern, splits=args.splits, kwaves=args.kwaves)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for pk in copies:
                    w4.linear(x[:M], pk, y=y[:M], kernel=kern, splits=args.splits, kwaves=args.kwaves)
            g.replay()
            torch.cuda.synchronize()
            # 20 repeats of at least 200 calls each; the figure is the median
            # of the repeats' per-call means
            replays = -(-200 // R)
            per_call = []
            for _ in range(20):
                s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s0.record()
                for _ in range(replays):
                    g.replay()
                s1.record()
                s1.synchronize()
                per_call.append(s0.elapsed_time(s1) * 1e3 / (R * replays))
            med = float(np.median(per_call))
            B, F = alg_bytes(M, N, K), alg_flops(M, N, K)
            t_roof = max(B / (HBM_PEAK_GBS * 1e9), F / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6
            print(json.dumps({"linear": name, "N": N, "K": K, "M": M, "us": round(med, 3),
                              "us_min": round(min(per_call), 3), "us_max": round(max(per_call), 3),
                              "protocol": f"median of 20 repeats x {R * replays} calls",
                              "tbps": round(B / (med * 1e-6) / 1e12, 4), "roofline_frac": round(t_roof / med, 4),
                              "mfma_util": round(F / (med * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
                              "plan": plan, "rotation_copies": R}), flush=True)
            del g
        del copies, base
        torch.cuda.empty_cache()


def floor_report(args):
    """Separate-launch floor: a plain 128-bit streaming read (w4_bench_read,
    graph-replayed over rotating buffers past the MALL) of each linear's packed
    bytes, an empty launch, and the sum of those reads over the linears of a
    pass -- the 561 separate linears, and the 321 with q|k|v and gate|up fused
    -- the least time any design that keeps one launch per linear can take,
    against the 8 TB/s roofline of the same bytes."""
    import torch

    import speculative_decoding_verification_w4a16_amd as w4
    import synth

    dev = "cuda:0"
    sink = torch.empty(w4.w4_bench_read_blocks(), dtype=torch.int32, device=dev)

    def timed(nbytes, copies):
        for b in copies[:2]:
            w4.w4_bench_read(b, nbytes, sink)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for b in copies:
                w4.w4_bench_read(b, nbytes, sink)
        g.replay()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(max(3, args.steps)):
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record()
            g.replay()
            s1.record()
            s1.synchronize()
            best = min(best, s0.elapsed_time(s1) * 1e3 / len(copies))
        del g
        return best

    tiny = [torch.zeros(16, dtype=torch.uint8, device=dev) for _ in range(200)]
    us_empty = timed(16, tiny)
    del tiny
    print(json.dumps({"launch": "w4_bench_read of 16 bytes", "us": round(us_empty, 3)}), flush=True)
    dims = {name: (N, K) for name, N, K in synth.LAYER_LINEARS}
    fused = [(f, sum(dims[n][0] for n in names), dims[names[0]][1]) for f, names in FUSED_GROUPS if len(names) > 1]
    shapes = list(synth.LAYER_LINEARS) + fused + [synth.LM_HEAD]
    floors = {}
    for name, N, K in shapes:
        nbytes = (int(N * K * 0.51953125) + 15) // 16 * 16
        R = max(2, int(args.rotate_gib * (1 << 30) // nbytes))
        copies = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(R)]
        for b in copies:
            b.fill_(1)
        us = timed(nbytes, copies)
        floors[name] = us
        print(json.dumps({"linear": name, "N": N, "K": K, "bytes": nbytes, "us": round(us, 3),
                          "tbps": round(nbytes / (us * 1e-6) / 1e12, 4), "rotation_copies": R}), flush=True)
        del copies
        torch.cuda.empty_cache()
    pass_us = synth.N_LAYERS * sum(floors[n] for n, _, _ in synth.LAYER_LINEARS) + floors["lm_head"]
    pass_bytes = synth.N_LAYERS * sum(N * K * 0.51953125 for _, N, K in synth.LAYER_LINEARS) + \
        synth.LM_HEAD[1] * synth.LM_HEAD[2] * 0.51953125
    print(json.dumps({"pass": "561 linears", "pass_floor_us": round(pass_us, 1), "pass_bytes": int(pass_bytes),
                      "floor_tbps": round(pass_bytes / (pass_us * 1e-6) / 1e12, 4),
                      "floor_roofline_frac": round(pass_bytes / (HBM_PEAK_GBS * 1e9) * 1e6 / pass_us, 4)}),
          flush=True)
    fused_us = synth.N_LAYERS * sum(floors[f] for f, _ in FUSED_GROUPS) + floors["lm_head"]
    print(json.dumps({"pass": "321 linears (q|k|v and gate|up fused)", "pass_floor_us": round(fused_us, 1),
                      "pass_bytes": int(pass_bytes),
                      "floor_tbps": round(pass_bytes / (fused_us * 1e-6) / 1e12, 4),
                      "floor_roofline_frac": round(pass_bytes / (HBM_PEAK_GBS * 1e9) * 1e6 / fused_us, 4)}),
          flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the verify linear is measured on one MI355X); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if args.shapes:
        shapes_report(args)
        return
    if args.floor:
        floor_report(args)
        return
    if args.curve_from:
        print(curve_tables(args.curve_from))
        return
    if args.trace_summary:
        print(json.dumps(trace_summary(args.trace_summary)))
        return
    if args.traffic_from:
        out = traffic_from_pmc(args.traffic_from[0], args.traffic_from[1], args.copy_calib or 1024,
                               os.path.join(ROOT, "profiles", "traffic.json"))
        print(json.dumps(out))
        return
    import torch

    import speculative_decoding_verification_w4a16_amd as w4
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.tree:
        w4.w4_init()
        print(json.dumps(tree_attention_bench(torch, w4, args)))
        return
    if args.tree_merge_sweep:
        w4.w4_init()
        tree_merge_sweep(torch, w4)
        return
    t_start = time.time()
    w4.w4_init()
    rng = np.random.default_rng(0)
    check_layers = sorted(int(v) for v in rng.choice(synth.N_LAYERS, 3, replace=False))
    n0 = int(rng.integers(0, (synth.LM_HEAD[1] - 512) // 8)) * 8
    keep = set(check_layers) | {0}
    packed, host = build_model(torch, w4, keep, keep_linears={(None, "lm_head")})
    t_model = time.time() - t_start
    log(f"[bench] model resident after {t_model:.1f} s; checked layers {check_layers}, lm_head cols {n0}..{n0 + 512}")

    dev = "cuda:0"
    if args.copy_calib:
        copy_calibration(torch, w4, args.copy_calib)
    specs = model_specs()

    # the dependent passes (the measured workload): the layer's projections
    # that share an input fused (q|k|v, gate|up), each linear reading its
    # producer's output
    fpk = fuse_projections(w4, packed)
    forced = {"auto": None, "persistent": w4.W4_PASS_PERSISTENT, "launches": w4.W4_PASS_LAUNCHES}[args.pass_mode]
    passes = {M: fused_dependent_pass(torch, w4, fpk, M, mode=forced if M <= 16 else None) for M in PASS_M}
    pass_bytes = {M: sum(alg_bytes(M, d["N"], d["K"], 2) for d in passes[M][3]) for M in PASS_M}
    pass_flops = {M: sum(alg_flops(M, d["N"], d["K"]) for d in passes[M][3]) for M in PASS_M}
    nlaunch = len(passes[PASS_M[0]][3])
    info = {M: w4.w4_pass_info(passes[M][0]) for M in PASS_M}
    for M in PASS_M:  # eager run once per M (also the graph's warm-up)
        w4.w4_pass_run(passes[M][0])
        w4.w4_pass_check(passes[M][0])
    graphs = {}
    cap = torch.cuda.Stream()
    for M in PASS_M:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            w4.w4_pass_run(passes[M][0])
        graphs[M] = g
    torch.cuda.synchronize()

    def step():
        for M in PASS_M:
            graphs[M].replay()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    for M in PASS_M:
        w4.w4_pass_check(passes[M][0])  # no dependency wait gave up in any replay
    step_bytes = sum(pass_bytes.values())
    value_tbs = step_bytes / (ms_per_step * 1e-3) / 1e12

    # per-M pass times (graph replays)
    def replay_us(g, reps):
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(reps):
            g.replay()
        s1.record()
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) * 1e3 / reps

    us_per_pass = {M: replay_us(graphs[M], max(3, args.steps)) for M in PASS_M}
    us_eager = {}
    for M in PASS_M:
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        w4.w4_pass_run(passes[M][0])
        s1.record()
        torch.cuda.synchronize()
        us_eager[M] = s0.elapsed_time(s1) * 1e3

    # the persistent pass kernel on the same fused pass where the library
    # chose per-linear launches (M <= 16), for comparison
    def pass_entry(handle, descs, outs, h0, g, seed):
        Mh = h0.shape[0]
        eb = sum(alg_bytes(Mh, d["N"], d["K"], 2) for d in descs)
        ef = sum(alg_flops(Mh, d["N"], d["K"]) for d in descs)
        eus = replay_us(g, max(3, args.steps))
        w4.w4_pass_check(handle)
        ent = {"us": round(eus, 1), "roofline_frac": round(max(eb / (HBM_PEAK_GBS * 1e9),
                                                               ef / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6 / eus, 4),
               "launches": 1 if w4.w4_pass_info(handle)["persistent"] else len(descs)}
        if not args.no_parity:
            h0.copy_(torch.from_numpy(synth.gen_x(h0.shape[0], h0.shape[1], seed_base=seed).view(np.int16)))
            for t in outs.values():
                t.fill_(0x7FC0)
            g.replay()
            w4.w4_pass_check(handle)
        return ent

    persistent_form, unfused, us_separate, sep_bytes = {}, {}, {}, {}
    if not args.headline_only:
        for M in PASS_M:
            if M > 16 or info[M]["persistent"]:
                continue
            handle, pouts, ph0, pdescs = fused_dependent_pass(torch, w4, fpk, M, mode=w4.W4_PASS_PERSISTENT)
            w4.w4_pass_run(handle)
            w4.w4_pass_check(handle)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                w4.w4_pass_run(handle)
            g.replay()
            torch.cuda.synchronize()
            ent = pass_entry(handle, pdescs, pouts, ph0, g, 2600)
            if not args.no_parity:
                ent["worst_err_over_bound"] = fused_dependent_parity(w4, host, pdescs, check_layers, n0)
            torch.cuda.synchronize()
            del g
            w4.w4_pass_destroy(handle)
            del pouts, pdescs, ph0
            persistent_form[M] = ent

        # the same dependent pass over the seven unfused linears of each layer
        # (561 linears), for comparison
        for M in PASS_M:
            handle, uouts, uh0, udescs = dependent_pass(torch, w4, packed, M)
            w4.w4_pass_run(handle)
            w4.w4_pass_check(handle)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                w4.w4_pass_run(handle)
            g.replay()
            torch.cuda.synchronize()
            ent = pass_entry(handle, udescs, uouts, uh0, g, 2700)
            if not args.no_parity:
                ent["worst_err_over_bound"] = dependent_pass_parity(torch, w4, host, udescs, check_layers, n0, M)
            torch.cuda.synchronize()
            del g
            w4.w4_pass_destroy(handle)
            del uouts, udescs, uh0
            unfused[M] = ent

        # the same linears as 561 independent launches (no dependencies, one input
        # per K, fp32 outputs): the structure of a launch per linear, for comparison
        xs = {K: torch.from_numpy(synth.gen_x(64, K).view(np.int16)).to(dev) for K in (8192, 28672)}
        ys = {N: torch.empty((64, N), dtype=torch.float32, device=dev) for N in (1024, 8192, 28672, 128256)}

        def descs_for(M):
            out = []
            for sp in specs:
                pk = packed[(sp["layer"], sp["name"])]
                out.append(dict(x=xs[sp["K"]][:M], qweight_t=pk.qweight_t, scales_t=pk.scales_t, zeros_t=pk.zeros_t,
                                y=ys[sp["N"]][:M], N=sp["N"], K=sp["K"]))
            return out

        sep_descs = {M: descs_for(M) for M in PASS_M}
        for M in PASS_M:
            w4.w4a16_verify_pass(sep_descs[M], M)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                w4.w4a16_verify_pass(sep_descs[M], M)
            g.replay()
            torch.cuda.synchronize()
            us_separate[M] = replay_us(g, max(3, args.steps))
            del g
        sep_bytes = {M: sum(alg_bytes(M, sp["N"], sp["K"]) for sp in specs) for M in PASS_M}

    # per-kernel roofline.  A pass in the persistent form is one launch of the
    # pass kernel (GEMV form at M = 1, MFMA form above); in the launch form
    # it is one launch per (fused) linear -- the GEMV at M = 1, the streaming
    # MFMA kernel at M = 2..14, the LDS-ring MFMA kernel above -- each with
    # its split-K reduction when K is split, and the unit is the linear
    # (averaged over the pass).  Durations come from the graph replays
    # (events on the replay stream).
    kernels = {}
    for M in PASS_M:
        if info[M]["persistent"]:
            name = "w4_pass_kernel<GEMV>" if M == 1 else "w4_pass_kernel<MFMA 16 rows>"
            launches = 1
        else:
            name = ("w4a16_gemv_kernel" if M == 1 else "w4a16_mfma_direct_kernel" if M <= 14
                    else "w4a16_mfma_lds_kernel<4, 4 or 8>")
            launches = nlaunch
        mean_us = us_per_pass[M] / launches
        bpl = pass_bytes[M] / launches
        achieved = bpl / (mean_us * 1e-6) / 1e9
        kernels[name] = {
            "M": M, "launches_per_pass": launches, "mean_launch_us": round(mean_us, 3),
            "alg_bytes_per_launch": int(bpl), "achieved_GBps": round(achieved, 1),
            "frac_hbm": round(achieved / HBM_PEAK_GBS, 4),
            "mfma_util": round(pass_flops[M] / launches / (mean_us * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
            "time_share_us": round(us_per_pass[M], 1)}
    dom = max(kernels, key=lambda k: kernels[k]["time_share_us"])
    dk = kernels[dom]
    traffic = traffic_from_profiles(dk["M"])
    roofline = {"bound": "hbm", "achieved": dk["achieved_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dk["achieved_GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom,
                "per_launch": ("alg_bytes_per_launch = 0.51953125 N K + 2 M K + 2 M N (bf16 output) summed over "
                               "the launch's linears: the 321 (fused) linears of the pass for the persistent pass "
                               "kernel, one linear (averaged over the pass, with its split-K reduction) for "
                               "per-linear launches; achieved = that / the launch's mean duration from the graph "
                               "replays")}

    fused = acceptance = tree = None
    if not args.no_extras and not args.headline_only:
        fused = fused_sweep(torch, w4, fpk, xs, host, check_layers, args)
        acceptance = acceptance_bench(torch, w4, args)
        tree = tree_attention_bench(torch, w4, args)

    ceiling = hbm_read_ceiling(torch, w4)
    parity = None
    if not args.no_parity and not args.headline_only:
        worst = {}
        for M in PASS_M:
            handle, outs, h0, pdescs = passes[M]
            h0.copy_(torch.from_numpy(synth.gen_x(M, h0.shape[1], seed_base=2500).view(np.int16)))
            for t in outs.values():
                t.fill_(0x7FC0)  # bf16 NaN: an output left unwritten, or read early, shows up
            graphs[M].replay()  # the captured pass, on a changed input
            w4.w4_pass_check(handle)
            worst[str(M)] = fused_dependent_parity(w4, host, pdescs, check_layers, n0)
        parity = {"layers": check_layers, "lm_head_cols": [n0, n0 + 512], "columns": "all (lm_head: the slice)",
                  "worst_err_over_bound": worst}
    cpu = None if args.no_cpu_baseline or args.headline_only else cpu_baseline(host)

    t_roof = {M: max(pass_bytes[M] / (HBM_PEAK_GBS * 1e9), pass_flops[M] / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6
              for M in PASS_M}
    out = {
        "metric": "int4-weight verify GEMM us/pass + HBM TB/s, Llama-3-70B shapes, M=1/5/64",
        "value": round(value_tbs, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian weights quantised to uint4 g=128, Gaussian bf16 activations)",
        "config": {"workload": "llama3-70b-w4a16-verify-sweep", "layers": 80, "weight_matrices": len(specs),
                   "linears_per_pass": nlaunch,
                   "projections": "q|k|v and gate|up fused (the layer's weights concatenated: N = 10240, 57344)",
                   "passes_per_step": list(PASS_M), "group": 128, "weight_bytes": int(sum(
                       s["N"] * s["K"] * 0.51953125 for s in specs)), "graph": True,
                   "dependencies": "each linear reads its producer's bf16 output (o: the q columns of qkv's, "
                                   "down: the gate columns of gate_up's)", "output": "bf16",
                   "launches_per_pass": {str(M): (1 if info[M]["persistent"] else nlaunch) for M in PASS_M},
                   "pass_mode": args.pass_mode},
        "us_per_pass": {str(M): round(us_per_pass[M], 1) for M in PASS_M},
        "us_per_pass_eager": {str(M): round(us_eager[M], 1) for M in PASS_M},
        "persistent_form": {"linears_per_pass": nlaunch,
                            "us_per_pass": {str(M): e["us"] for M, e in persistent_form.items()},
                            "roofline_frac_per_pass": {str(M): e["roofline_frac"] for M, e in persistent_form.items()},
                            "worst_err_over_bound": {str(M): e.get("worst_err_over_bound")
                                                     for M, e in persistent_form.items()}} if persistent_form else None,
        "unfused_dependent": {"linears_per_pass": len(specs),
                              "us_per_pass": {str(M): unfused[M]["us"] for M in PASS_M},
                              "roofline_frac_per_pass": {str(M): unfused[M]["roofline_frac"] for M in PASS_M},
                              "launches_per_pass": {str(M): unfused[M]["launches"] for M in PASS_M},
                              "worst_err_over_bound": {str(M): unfused[M].get("worst_err_over_bound")
                                                       for M in PASS_M}} if unfused else None,
        "separate_launches": {"us_per_pass": {str(M): round(us_separate[M], 1) for M in PASS_M},
                              "roofline_frac_per_pass": {str(M): round(max(
                                  sep_bytes[M] / (HBM_PEAK_GBS * 1e9),
                                  pass_flops[M] / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6 / us_separate[M], 4)
                                  for M in PASS_M}} if us_separate else None,
        "tbps_per_pass": {str(M): round(pass_bytes[M] / (us_per_pass[M] * 1e-6) / 1e12, 4) for M in PASS_M},
        "roofline_frac_per_pass": {str(M): round(t_roof[M] / us_per_pass[M], 4) for M in PASS_M},
        "t_over_t1": {str(M): round(us_per_pass[M] / us_per_pass[1], 4) for M in PASS_M},
        "hbm_read_ceiling_tbps": round(ceiling / 1000, 4),
        "roofline": roofline,
        "kernels": kernels,
        "fused": fused,
        "acceptance": acceptance,
        "tree_attention": tree,
        "cost_model": cost_table(us_per_pass),
        "cost_model_fused": cost_table(fused["us_per_pass"]) if fused else None,
        "cpu_baseline": cpu,
        "parity": parity,
        "setup_s": round(t_model, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
