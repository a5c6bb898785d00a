"""Python binding of libw4a16.so, the MI355X W4A16 verify-linear library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/w4a16.h``.  The functions
here carry the C names, take torch tensors (device memory from PyTorch-ROCm)
or raw integer addresses, pass the current HIP stream of the tensor's
device, and raise ``W4Error`` on a nonzero status.  Importing the package
fails loudly when the built library is missing; there is no fallback path.

Build the library with ``python speculative_decoding_verification_w4a16_amd/build.py``
(or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# W4A16_LIB selects another build of the same library (the tests use it to
# load the host-sanitizer build); by default the in-tree libw4a16.so.
LIB_PATH = os.environ.get("W4A16_LIB") or os.path.join(HERE, "libw4a16.so")

W4_OK, W4_ERR_INVALID, W4_ERR_UNSUPPORTED, W4_ERR_HIP, W4_ERR_TIMEOUT = 0, 1, 2, 3, 4
W4_PASS_MAX_DEPS = 4
W4_PASS_AUTO, W4_PASS_PERSISTENT, W4_PASS_LAUNCHES = 0, 1, 2
W4_KERNEL_AUTO, W4_KERNEL_GEMV, W4_KERNEL_MFMA = 0, 1, 2
W4_OUT_F32, W4_OUT_BF16 = 0, 1
GROUP = 128
MAX_M = 64

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python speculative_decoding_verification_w4a16_amd/build.py`")

# PyTorch-ROCm ships its own libamdhip64 (same soname as /opt/rocm's, but
# loaded under another file name).  Loading this library first would bring in
# /opt/rocm's runtime and torch would then load a second one, which cannot
# open the device.  Importing torch first makes both use torch's runtime.
try:
    import torch as _torch  # noqa: F401
except ImportError:  # pragma: no cover - the library itself does not need torch
    _torch = None

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t


class W4LinearDesc(ctypes.Structure):
    _fields_ = [("x", _vp), ("qweight_t", _vp), ("scales_t", _vp), ("zeros_t", _vp), ("y", _vp), ("N", _i),
                ("K", _i)]


class W4PassLinear(ctypes.Structure):
    _fields_ = [("x", _vp), ("qweight_t", _vp), ("scales_t", _vp), ("zeros_t", _vp), ("y", _vp), ("y_bf16", _vp),
                ("alpha", ctypes.c_float), ("N", _i), ("K", _i), ("ndeps", _i), ("deps", _i * 4), ("ldx", _i)]


def _sig(name, args, res=_i):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_c = {
    "w4_status_str": _sig("w4_status_str", [_i], ctypes.c_char_p),
    "w4_init": _sig("w4_init", []),
    "w4_last_error": _sig("w4_last_error", [], ctypes.c_char_p),
    "w4_repacked_sizes": _sig("w4_repacked_sizes", [_i, _i, _i, ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                                    ctypes.POINTER(_sz)]),
    "w4_repack": _sig("w4_repack", [_vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "w4a16_linear": _sig("w4a16_linear", [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]),
    "w4a16_linear_cfg": _sig("w4a16_linear_cfg", [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _i, _i, _vp]),
    "w4a16_linear_out": _sig("w4a16_linear_out", [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _i, _i, _i, _vp]),
    "w4a16_linear_out_noalloc": _sig("w4a16_linear_out_noalloc",
                                     [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _i, _i, _i, _vp]),
    "w4a16_linear_tune": _sig("w4a16_linear_tune",
                              [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _vp]),
    "w4a16_plan": _sig("w4a16_plan", [_i, _i, _i, _i, _i, _i, _i] + [ctypes.POINTER(_i)] * 6),
    "w4a16_verify_pass": _sig("w4a16_verify_pass", [ctypes.POINTER(W4LinearDesc), _i, _i, _i, _vp]),
    "w4_unpack": _sig("w4_unpack", [_vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    "w4_pass_create": _sig("w4_pass_create", [ctypes.POINTER(W4PassLinear), _i, _i, _i, ctypes.POINTER(_vp)]),
    "w4_pass_create_mode": _sig("w4_pass_create_mode",
                                [ctypes.POINTER(W4PassLinear), _i, _i, _i, _i, ctypes.POINTER(_vp)]),
    "w4_pass_run": _sig("w4_pass_run", [_vp, _vp]),
    "w4_pass_check": _sig("w4_pass_check", [_vp, _vp]),
    "w4_pass_info": _sig("w4_pass_info", [_vp, ctypes.POINTER(_i), ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    "w4_pass_set_spin_limit": _sig("w4_pass_set_spin_limit", [_vp, ctypes.c_uint32]),
    "w4_pass_destroy": _sig("w4_pass_destroy", [_vp]),
    "w4_bench_read": _sig("w4_bench_read", [_vp, _sz, _vp, _vp]),
    "w4_bench_read_blocks": _sig("w4_bench_read_blocks", []),
    "w4_bench_copy": _sig("w4_bench_copy", [_vp, _vp, _sz, _vp]),
    "w4_accept_greedy": _sig("w4_accept_greedy", [_vp, _vp, _i, _i, _vp, _vp]),
    "w4_accept_sample": _sig("w4_accept_sample", [_vp, _vp, _vp, _vp, _i, _i, _vp, _vp]),
    "w4_tree_attention": _sig("w4_tree_attention",
                              [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, ctypes.c_float, _vp, _vp]),
    "w4_tree_attention_ex": _sig("w4_tree_attention_ex",
                                 [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, ctypes.c_float, _i, _vp, _vp]),
    "w4_tree_attention_plan": _sig("w4_tree_attention_plan",
                                   [_i, _i, _i, _i, _i, ctypes.POINTER(_i), ctypes.POINTER(_i)]),
}


class W4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        detail = f" [{w4_last_error()}]" if status == W4_ERR_HIP else ""
        super().__init__(f"{where}: {w4_status_str(status)}{detail}")
        self.status = status


def exported_symbols():
    """Names of the C entry points this binding wraps (all must be exported)."""
    return sorted(_c)


def _ptr(t):
    """Device address of a tensor (or an int address, or None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    dev = None
    for t in tensors:
        if t is not None and not isinstance(t, int) and t.is_cuda:
            dev = t.device
            break
    if dev is None:
        return None
    return torch.cuda.current_stream(dev).cuda_stream


def _check(rc, where):
    if rc != W4_OK:
        raise W4Error(rc, where)


def w4_status_str(status: int) -> str:
    return _c["w4_status_str"](status).decode()


def w4_last_error() -> str:
    return _c["w4_last_error"]().decode()


def w4_init() -> None:
    _check(_c["w4_init"](), "w4_init")


def w4_repacked_sizes(N: int, K: int, group: int = GROUP):
    q, s, z = _sz(), _sz(), _sz()
    _check(_c["w4_repacked_sizes"](N, K, group, ctypes.byref(q), ctypes.byref(s), ctypes.byref(z)),
           "w4_repacked_sizes")
    return q.value, s.value, z.value


def w4_repack(qweight, scales, zeros, N, K, group, qweight_t, scales_t, zeros_t, stream=None):
    st = _stream(stream, qweight, qweight_t)
    _check(_c["w4_repack"](_ptr(qweight), _ptr(scales), _ptr(zeros), N, K, group, _ptr(qweight_t), _ptr(scales_t),
                           _ptr(zeros_t), st), "w4_repack")


def w4a16_linear(x, qweight_t, scales_t, zeros_t, M, N, K, group, y, stream=None):
    st = _stream(stream, x, y)
    _check(_c["w4a16_linear"](_ptr(x), _ptr(qweight_t), _ptr(scales_t), _ptr(zeros_t), M, N, K, group, _ptr(y), st),
           "w4a16_linear")


def w4a16_linear_cfg(x, qweight_t, scales_t, zeros_t, M, N, K, group, y, kernel=W4_KERNEL_AUTO, splits=0,
                     stream=None):
    st = _stream(stream, x, y)
    _check(_c["w4a16_linear_cfg"](_ptr(x), _ptr(qweight_t), _ptr(scales_t), _ptr(zeros_t), M, N, K, group, _ptr(y),
                                  kernel, splits, st), "w4a16_linear_cfg")


def w4a16_linear_out(x, qweight_t, scales_t, zeros_t, M, N, K, group, y, out_dtype=W4_OUT_F32,
                     kernel=W4_KERNEL_AUTO, splits=0, stream=None):
    st = _stream(stream, x, y)
    _check(_c["w4a16_linear_out"](_ptr(x), _ptr(qweight_t), _ptr(scales_t), _ptr(zeros_t), M, N, K, group, _ptr(y),
                                  out_dtype, kernel, splits, st), "w4a16_linear_out")


def w4a16_linear_out_noalloc(x, qweight_t, scales_t, zeros_t, M, N, K, group, y, out_dtype=W4_OUT_F32,
                             kernel=W4_KERNEL_AUTO, splits=0, stream=None):
    st = _stream(stream, x, y)
    _check(_c["w4a16_linear_out_noalloc"](_ptr(x), _ptr(qweight_t), _ptr(scales_t), _ptr(zeros_t), M, N, K, group,
                                          _ptr(y), out_dtype, kernel, splits, st), "w4a16_linear_out_noalloc")


def w4a16_linear_tune(x, qweight_t, scales_t, zeros_t, M, N, K, group, y, out_dtype=W4_OUT_F32,
                      kernel=W4_KERNEL_AUTO, splits=0, kwaves=0, stream=None):
    st = _stream(stream, x, y)
    _check(_c["w4a16_linear_tune"](_ptr(x), _ptr(qweight_t), _ptr(scales_t), _ptr(zeros_t), M, N, K, group,
                                   _ptr(y), out_dtype, kernel, splits, kwaves, st), "w4a16_linear_tune")


def w4a16_plan(M, N, K, group=GROUP, kernel=W4_KERNEL_AUTO, splits=0, kwaves=0) -> dict:
    outs = [_i() for _ in range(6)]
    _check(_c["w4a16_plan"](M, N, K, group, kernel, splits, kwaves, *[ctypes.byref(o) for o in outs]),
           "w4a16_plan")
    return dict(zip(("kernel", "splits", "kwaves", "grid", "block", "lds"), (o.value for o in outs)))


def w4a16_verify_pass(linears, M, group=GROUP, stream=None):
    """`linears`: sequence of dicts with x, qweight_t, scales_t, zeros_t, y, N, K."""
    arr = (W4LinearDesc * max(1, len(linears)))()
    for i, d in enumerate(linears):
        arr[i] = W4LinearDesc(_ptr(d["x"]), _ptr(d["qweight_t"]), _ptr(d["scales_t"]), _ptr(d["zeros_t"]),
                              _ptr(d["y"]), d["N"], d["K"])
    first = linears[0]["y"] if linears else None
    st = _stream(stream, first)
    _check(_c["w4a16_verify_pass"](arr, len(linears), M, group, st), "w4a16_verify_pass")


def _pass_array(linears):
    n = len(linears)
    arr = (W4PassLinear * max(1, n))()
    for i, d in enumerate(linears):
        deps = list(d.get("deps", ()))
        arr[i] = W4PassLinear(_ptr(d["x"]), _ptr(d["qweight_t"]), _ptr(d["scales_t"]), _ptr(d["zeros_t"]),
                              _ptr(d.get("y")), _ptr(d.get("y_bf16")), float(d.get("alpha", 1.0)), d["N"], d["K"],
                              len(deps), (_i * 4)(*(deps + [0] * (4 - len(deps)))[:4]), int(d.get("ldx", 0)))
    return arr, n


def w4_pass_create(linears, M, group=GROUP):
    """`linears`: sequence of dicts with x, qweight_t, scales_t, zeros_t, y
    (or None), y_bf16 (or None), N, K, and optionally alpha (1.0), deps
    (indices of earlier entries) and ldx (elements between rows of x; 0, the
    default, means K).  The library chooses the form.  Returns the pass
    handle (an int)."""
    arr, n = _pass_array(linears)
    out = _vp()
    _check(_c["w4_pass_create"](arr, n, M, group, ctypes.byref(out)), "w4_pass_create")
    return out.value


def w4_pass_create_mode(linears, M, mode, group=GROUP):
    """w4_pass_create with the form chosen: `mode` is W4_PASS_AUTO,
    W4_PASS_PERSISTENT or W4_PASS_LAUNCHES."""
    arr, n = _pass_array(linears)
    out = _vp()
    _check(_c["w4_pass_create_mode"](arr, n, M, group, mode, ctypes.byref(out)), "w4_pass_create_mode")
    return out.value


def w4_pass_run(handle, stream=None):
    if stream is None:
        import torch

        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(_c["w4_pass_run"](handle, stream), "w4_pass_run")


def w4_pass_check(handle, stream=None):
    """Synchronize `stream`; raise W4Error (W4_ERR_TIMEOUT) if a dependency
    wait of the runs since the last check gave up."""
    if stream is None:
        import torch

        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(_c["w4_pass_check"](handle, stream), "w4_pass_check")


def w4_pass_info(handle) -> dict:
    outs = [_i() for _ in range(3)]
    _check(_c["w4_pass_info"](handle, *[ctypes.byref(o) for o in outs]), "w4_pass_info")
    return dict(zip(("persistent", "grid", "units"), (o.value for o in outs)))


def w4_pass_set_spin_limit(handle, polls):
    _check(_c["w4_pass_set_spin_limit"](handle, polls), "w4_pass_set_spin_limit")


def w4_pass_destroy(handle):
    _check(_c["w4_pass_destroy"](handle), "w4_pass_destroy")


def w4_unpack(qweight_t, zeros_t, N, K, group, q_out, z_out, stream=None):
    st = _stream(stream, qweight_t, q_out)
    _check(_c["w4_unpack"](_ptr(qweight_t), _ptr(zeros_t), N, K, group, _ptr(q_out), _ptr(z_out), st), "w4_unpack")


def w4_bench_read_blocks() -> int:
    return int(_c["w4_bench_read_blocks"]())


def w4_bench_read(buf, nbytes, sink, stream=None):
    st = _stream(stream, buf)
    _check(_c["w4_bench_read"](_ptr(buf), nbytes, _ptr(sink), st), "w4_bench_read")


def w4_accept_greedy(logits, draft, K, V, out, stream=None):
    st = _stream(stream, logits, out)
    _check(_c["w4_accept_greedy"](_ptr(logits), _ptr(draft), K, V, _ptr(out), st), "w4_accept_greedy")


def w4_accept_sample(logits, draft_logits, draft, u, K, V, out, stream=None):
    st = _stream(stream, logits, out)
    _check(_c["w4_accept_sample"](_ptr(logits), _ptr(draft_logits), _ptr(draft), _ptr(u), K, V, _ptr(out), st),
           "w4_accept_sample")


def accept(logits, draft, draft_logits=None, u=None, out=None, stream=None):
    """Acceptance step on device tensors: logits [K+1, V] fp32, draft [K]
    int32, and for the sampled step draft_logits [K, V] fp32 and u [K+1] fp32.
    Returns an int32 tensor [2]: (drafted tokens accepted, next token)."""
    import torch

    if logits.dim() != 2 or logits.shape[0] < 1:
        raise ValueError(f"logits: expected [K+1, V], got shape {tuple(logits.shape)}")
    K, V = logits.shape[0] - 1, logits.shape[1]
    dev = logits.device
    _require("logits", logits, (K + 1, V), (4,))
    if logits.dtype != torch.float32:
        raise ValueError(f"logits: expected float32, got {logits.dtype}")
    _require("draft", draft, (K,), (4,))
    if draft.dtype != torch.int32:
        raise ValueError(f"draft: expected int32, got {draft.dtype}")
    if (draft_logits is None) != (u is None):
        raise ValueError("the sampled step needs both draft_logits and u")
    if draft_logits is not None:
        _require("draft_logits", draft_logits, (K, V), (4,))
        _require("u", u, (K + 1,), (4,))
        if draft_logits.dtype != torch.float32 or u.dtype != torch.float32:
            raise ValueError("draft_logits and u must be float32")
        _on_device(dev, draft_logits=draft_logits, u=u)
    if out is not None:
        _require("out", out, (2,), (4,))
        _on_device(dev, out=out)
    _on_device(dev, logits=logits, draft=draft)
    if out is None:
        out = torch.empty(2, dtype=torch.int32, device=dev)
    if draft_logits is None:
        w4_accept_greedy(logits, draft, K, V, out, stream)
    else:
        w4_accept_sample(logits, draft_logits, draft, u, K, V, out, stream)
    return out


def w4_tree_attention(q, k_cache, v_cache, k_draft, v_draft, masks, M, L, num_heads, num_kv_heads, head_dim,
                      scale, out, stream=None):
    st = _stream(stream, q, out)
    _check(_c["w4_tree_attention"](_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_draft), _ptr(v_draft), _ptr(masks),
                                   M, L, num_heads, num_kv_heads, head_dim, scale, _ptr(out), st),
           "w4_tree_attention")


def w4_tree_attention_ex(q, k_cache, v_cache, k_draft, v_draft, masks, M, L, num_heads, num_kv_heads, head_dim,
                         scale, merge, out, stream=None):
    st = _stream(stream, q, out)
    _check(_c["w4_tree_attention_ex"](_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_draft), _ptr(v_draft),
                                      _ptr(masks), M, L, num_heads, num_kv_heads, head_dim, scale, merge, _ptr(out),
                                      st),
           "w4_tree_attention_ex")


TREE_MERGE_AUTO, TREE_MERGE_LAUNCH, TREE_MERGE_LAST = 0, 1, 2


def w4_tree_attention_plan(M, L, num_heads, num_kv_heads, merge=TREE_MERGE_AUTO):
    """(key splits, merge used) of a tree attention call of that shape."""
    splits, used = ctypes.c_int(0), ctypes.c_int(0)
    _check(_c["w4_tree_attention_plan"](M, L, num_heads, num_kv_heads, merge, ctypes.byref(splits),
                                        ctypes.byref(used)),
           "w4_tree_attention_plan")
    return splits.value, used.value


def tree_attention(q, k_cache, v_cache, k_draft, v_draft, masks, scale=0.0, out=None, stream=None,
                   merge=TREE_MERGE_AUTO):
    """Tree-draft verify attention on device tensors: q [M, Hq, 128], caches
    [L, Hkv, 128] and draft keys/values [M, Hkv, 128] as bf16 (or int16 bf16
    bits), masks [M] int64 (uint64 bit patterns).  Returns fp32 [M, Hq, 128].
    merge: how the key splits are merged (TREE_MERGE_AUTO, _LAUNCH, _LAST)."""
    import torch

    if q.dim() != 3 or k_cache.dim() != 3 or k_draft.dim() != 3:
        raise ValueError("q [M, Hq, D], caches [L, Hkv, D] and draft keys/values [M, Hkv, D] are 3-D")
    M, Hq, D = q.shape
    L, Hkv = k_cache.shape[0], k_draft.shape[1]
    dev = q.device
    _require("q", q, (M, Hq, D), (2,))
    _require("k_cache", k_cache, (L, Hkv, D), (2,))
    _require("v_cache", v_cache, (L, Hkv, D), (2,))
    _require("k_draft", k_draft, (M, Hkv, D), (2,))
    _require("v_draft", v_draft, (M, Hkv, D), (2,))
    _require("masks", masks, (M,), (8,))
    if out is not None:
        _require("out", out, (M, Hq, D), (4,))
        if out.dtype != torch.float32:
            raise ValueError(f"out: expected float32, got {out.dtype}")
        _on_device(dev, out=out)
    _on_device(dev, q=q, k_cache=k_cache, v_cache=v_cache, k_draft=k_draft, v_draft=v_draft, masks=masks)
    if out is None:
        out = torch.empty((M, Hq, D), dtype=torch.float32, device=dev)
    w4_tree_attention_ex(q, k_cache if L else None, v_cache if L else None, k_draft, v_draft, masks, M, L, Hq, Hkv,
                         D, scale, merge, out, stream)
    return out


def w4_bench_copy(dst, src, nbytes, stream=None):
    st = _stream(stream, dst)
    _check(_c["w4_bench_copy"](_ptr(dst), _ptr(src), nbytes, st), "w4_bench_copy")


# ---------------------------------------------------------------------------
# torch-tensor conveniences (allocation + the calls above)
# ---------------------------------------------------------------------------

def _require(name, t, shape, itemsizes):
    """Raise ValueError unless `t` is a contiguous tensor of `shape` whose
    element size is one of `itemsizes`.  The C ABI takes raw addresses and
    trusts the sizes it is given, so the conveniences check every tensor
    they hand over (then _on_device checks where they live)."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.element_size() not in itemsizes:
        raise ValueError(f"{name}: {t.dtype} has {t.element_size()}-byte elements, expected {itemsizes}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _on_device(device, **tensors):
    """Raise ValueError unless every tensor is a GPU tensor on `device`."""
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError(f"{name}: expected a GPU tensor, got one on {t.device}")
        if t.device != device:
            raise ValueError(f"{name}: on {t.device}, expected {device}")


class PackedLinear:
    """Tile-layout weights of one (N, K) linear on a device."""

    def __init__(self, qweight_t, scales_t, zeros_t, N, K, group=GROUP):
        self.qweight_t, self.scales_t, self.zeros_t = qweight_t, scales_t, zeros_t
        self.N, self.K, self.group = N, K, group

    @property
    def nbytes(self) -> int:
        return self.qweight_t.numel() * 4 + self.scales_t.numel() * 2 + self.zeros_t.numel() * 2


def repack(qweight, scales, zeros, N, K, group=GROUP, stream=None) -> PackedLinear:
    """Device canonical tensors (int32, int16/uint16 bits, int32) -> PackedLinear."""
    import torch

    dev = qweight.device
    _require("qweight", qweight, (K // 8, N), (4,))
    _require("scales", scales, (K // group, N), (2,))
    _require("zeros", zeros, (K // group, N // 8), (4,))
    _on_device(dev, qweight=qweight, scales=scales, zeros=zeros)
    qb, sb, zb = w4_repacked_sizes(N, K, group)
    qt = torch.empty(qb // 4, dtype=torch.int32, device=dev)
    st = torch.empty(sb // 2, dtype=torch.int16, device=dev)
    zt = torch.empty(zb // 2, dtype=torch.int16, device=dev)
    w4_repack(qweight, scales, zeros, N, K, group, qt, st, zt, stream)
    return PackedLinear(qt, st, zt, N, K, group)


def linear(x, w: PackedLinear, y=None, kernel=W4_KERNEL_AUTO, splits=0, stream=None, out_bf16=False, kwaves=0):
    """y[M, N] = x[M, K] (bf16 tensor or int16 bf16 bits) . dequant(w): fp32,
    or bf16 bit patterns (int16 tensor) with out_bf16."""
    import torch

    if x.dim() != 2:
        raise ValueError(f"x: expected [M, K], got shape {tuple(x.shape)}")
    M = x.shape[0]
    _require("x", x, (M, w.K), (2,))
    qb, sb, zb = w4_repacked_sizes(w.N, w.K, w.group)
    _require("qweight_t", w.qweight_t, (qb // 4,), (4,))
    _require("scales_t", w.scales_t, (sb // 2,), (2,))
    _require("zeros_t", w.zeros_t, (zb // 2,), (2,))
    if y is not None:
        _require("y", y, (M, w.N), (2,) if out_bf16 else (4,))
        if not out_bf16 and y.dtype != torch.float32:
            raise ValueError(f"y: fp32 output needs a float32 tensor, got {y.dtype}")
    _on_device(x.device, x=x, qweight_t=w.qweight_t, scales_t=w.scales_t, zeros_t=w.zeros_t)
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.int16 if out_bf16 else torch.float32, device=x.device)
    else:
        _on_device(x.device, y=y)
    w4a16_linear_tune(x, w.qweight_t, w.scales_t, w.zeros_t, M, w.N, w.K, w.group, y,
                      W4_OUT_BF16 if out_bf16 else W4_OUT_F32, kernel, splits, kwaves, stream)
    return y


def concat_packed(parts) -> PackedLinear:
    """One linear computing the column concatenation of `parts` (same K and
    group, every N a multiple of 64): the tile layout is chunk-major, so the
    fused arrays are the parts' arrays end to end (a device copy)."""
    import torch

    K, group = parts[0].K, parts[0].group
    for p in parts:
        if p.K != K or p.group != group or p.N % 64 != 0:
            raise ValueError("concat_packed needs equal K and group and every N a multiple of 64")
    return PackedLinear(torch.cat([p.qweight_t for p in parts]), torch.cat([p.scales_t for p in parts]),
                        torch.cat([p.zeros_t for p in parts]), sum(p.N for p in parts), K, group)
