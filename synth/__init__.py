"""Seeded synthetic inputs for the W4A16 verify linear.

This module makes the inputs that both sides consume -- quantised Gaussian
weights in the canonical packed uint4 format and Gaussian bf16 activations --
and nothing else.  It holds none of the verify GEMM's arithmetic: no
unpacking, no dequantisation and no products.  The heavy lifting is in
``gen.c`` (Philox4x64-10 + Box-Muller + round-to-nearest min/max quantiser),
built with gcc into ``libw4synth.so`` next to this file.

Canonical packed format (the oracle's input and the library's repack input):

* ``qweight`` int32 ``[K/8, N]``: bits ``[4i, 4i+4)`` of word ``(j, n)`` hold
  ``q[8j+i, n]`` (low nibble first);
* ``scales`` uint16 ``[K/g, N]``: fp16 bit patterns;
* ``zeros`` int32 ``[K/g, N/8]``: bits ``[4i, 4i+4)`` of word ``(G, j)`` hold
  ``z[G, 8j+i]``;
* ``x`` uint16 ``[M, K]``: bf16 bit patterns, row-major.

Seeds (the workload recipe): tiny linear seed 0; the seven decoder linears
q, k, v, o, gate, up, down use ``1000 + idx``; layer ``L`` of the full-model
sweep uses ``10000 + 7 L + idx`` and its lm_head ``20000``; activation row
``i`` for hidden size 8192 is stream ``2000 + i`` and for 28672 is
``3000 + i`` (the tiny linear's rows use ``100 + i``), so the M-row input is
the first M rows of one table.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libw4synth.so")
_SRC = os.path.join(_HERE, "gen.c")
_lib = None

GROUP = 128
W_STD = 0.02

# the seven linears of one Llama-3-70B-shaped decoder layer: (name, N, K)
LAYER_LINEARS = (
    ("q", 8192, 8192),
    ("k", 1024, 8192),
    ("v", 1024, 8192),
    ("o", 8192, 8192),
    ("gate", 28672, 8192),
    ("up", 28672, 8192),
    ("down", 8192, 28672),
)
LM_HEAD = ("lm_head", 128256, 8192)
N_LAYERS = 80
TINY = ("tiny", 256, 512)


def build(force: bool = False) -> str:
    """Compile gen.c into libw4synth.so with gcc (seconds)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, u64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_float
        lib.w4s_gen_linear.argtypes = [u64, f32, i32, i32, i32, vp, vp, vp, i32]
        lib.w4s_gen_linear.restype = i32
        lib.w4s_quantize.argtypes = [vp, i32, i32, i32, vp, vp, vp, i32]
        lib.w4s_quantize.restype = i32
        lib.w4s_gen_x.argtypes = [u64, i32, i32, i32, vp]
        lib.w4s_gen_x.restype = None
        lib.w4s_normals.argtypes = [u64, u64, ctypes.c_size_t, f32, vp]
        lib.w4s_normals.restype = None
        lib.w4s_philox_block.argtypes = [u64, u64, u64, vp]
        lib.w4s_philox_block.restype = None
        lib.w4s_f32_to_f16.argtypes = [f32]
        lib.w4s_f32_to_f16.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def alloc_linear(N: int, K: int, group: int = GROUP, pinned: bool = False):
    """Empty canonical arrays for an (N, K) linear (numpy, optionally pinned torch)."""
    shapes = {"qweight": ((K // 8, N), np.int32), "scales": ((K // group, N), np.uint16),
              "zeros": ((K // group, N // 8), np.int32)}
    if not pinned:
        return {k: np.empty(s, d) for k, (s, d) in shapes.items()}
    import torch
    tdt = {np.int32: torch.int32, np.uint16: torch.int16}
    out = {}
    for k, (s, d) in shapes.items():
        t = torch.empty(s, dtype=tdt[d], pin_memory=True)
        out[k] = t.numpy().view(d)
    return out


def gen_linear(seed: int, N: int, K: int, group: int = GROUP, std: float = W_STD, out=None,
               nthreads: int | None = None) -> dict:
    """Gaussian weights N(0, std^2) of stream `seed`, quantised and packed.

    Returns a dict with ``qweight``, ``scales``, ``zeros`` numpy arrays."""
    if N % 8 or K % group or K % 8:
        raise ValueError("need N % 8 == 0 and K % group == 0")
    lib = _load()
    arrs = out if out is not None else alloc_linear(N, K, group)
    rc = lib.w4s_gen_linear(seed, std, N, K, group, arrs["qweight"].ctypes.data, arrs["scales"].ctypes.data,
                            arrs["zeros"].ctypes.data, nthreads or _threads())
    if rc != 0:
        raise RuntimeError("w4s_gen_linear failed")
    return arrs


def quantize(W: np.ndarray, group: int = GROUP) -> dict:
    """Quantise and pack a caller-supplied fp32 W [N, K] (row n = output column n)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    if N % 8 or K % group or K % 8:
        raise ValueError("need N % 8 == 0 and K % group == 0")
    lib = _load()
    arrs = alloc_linear(N, K, group)
    rc = lib.w4s_quantize(W.ctypes.data, N, K, group, arrs["qweight"].ctypes.data, arrs["scales"].ctypes.data,
                          arrs["zeros"].ctypes.data, _threads())
    if rc != 0:
        raise RuntimeError("w4s_quantize failed")
    return arrs


def normals(seed: int, count: int, scale: float = 1.0, start: int = 0) -> np.ndarray:
    """Elements [start, start+count) of stream `seed`, times `scale` (fp32)."""
    out = np.empty(count, np.float32)
    _load().w4s_normals(seed, start, count, scale, out.ctypes.data)
    return out


def weights_fp32(seed: int, N: int, K: int, std: float = W_STD) -> np.ndarray:
    """The unquantised W [N, K] that gen_linear(seed, N, K) quantises."""
    return normals(seed, N * K, std).reshape(N, K)


def x_seed_base(K: int) -> int:
    return {8192: 2000, 28672: 3000}.get(K, 100)


def gen_x(M: int, K: int, seed_base: int | None = None, row0: int = 0) -> np.ndarray:
    """Activations: row i is stream (seed_base + row0 + i), N(0,1) rounded to bf16 bits [M, K]."""
    if seed_base is None:
        seed_base = x_seed_base(K)
    out = np.empty((M, K), np.uint16)
    if M > 0 and K > 0:
        _load().w4s_gen_x(seed_base, row0, M, K, out.ctypes.data)
    return out


def philox_block(key0: int, key1: int, block: int) -> np.ndarray:
    out = np.empty(4, np.uint64)
    _load().w4s_philox_block(key0, key1, block, out.ctypes.data)
    return out


def f32_to_f16_bits(v: float) -> int:
    return int(_load().w4s_f32_to_f16(v))


def pack_q(q: np.ndarray) -> np.ndarray:
    """Pack uint4 codes q [K, N] (values 0..15) into canonical qweight int32 [K/8, N]."""
    q = np.asarray(q, dtype=np.uint32)
    K, N = q.shape
    if K % 8:
        raise ValueError("K % 8 != 0")
    q8 = q.reshape(K // 8, 8, N)
    word = np.zeros((K // 8, N), np.uint32)
    for i in range(8):
        word |= (q8[:, i, :] & 0xF) << np.uint32(4 * i)
    return word.view(np.int32)


def pack_z(z: np.ndarray) -> np.ndarray:
    """Pack uint4 zero points z [K/g, N] into canonical zeros int32 [K/g, N/8]."""
    z = np.asarray(z, dtype=np.uint32)
    G, N = z.shape
    if N % 8:
        raise ValueError("N % 8 != 0")
    z8 = z.reshape(G, N // 8, 8)
    word = np.zeros((G, N // 8), np.uint32)
    for i in range(8):
        word |= (z8[:, :, i] & 0xF) << np.uint32(4 * i)
    return word.view(np.int32)


def pack_linear(q: np.ndarray, z: np.ndarray, s_bits: np.ndarray) -> dict:
    """Canonical arrays from explicit codes q [K, N], zeros z [K/g, N], fp16 scale bits [K/g, N]."""
    return {"qweight": pack_q(q), "scales": np.ascontiguousarray(s_bits, dtype=np.uint16), "zeros": pack_z(z)}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even), returning the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)
