"""Helpers shared by the GPU tests: moving canonical arrays to the device,
repacking through the library and running the verify linear."""
from __future__ import annotations

import numpy as np

DEV = "cuda:0"


def torch_mod():
    import torch

    return torch


def to_dev(arr: np.ndarray):
    torch = torch_mod()
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint8:
        pass
    return torch.from_numpy(a).to(DEV)


def packed(lin: dict, N: int, K: int):
    import speculative_decoding_verification_w4a16_amd as w4

    return w4.repack(to_dev(lin["qweight"]), to_dev(lin["scales"]), to_dev(lin["zeros"]), N, K)


def run_linear(x_bits: np.ndarray, pk, kernel=0, splits=0, y=None) -> np.ndarray:
    import speculative_decoding_verification_w4a16_amd as w4

    torch = torch_mod()
    xd = to_dev(x_bits)
    out = w4.linear(xd, pk, y=y, kernel=kernel, splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def unpack_dev(pk):
    import speculative_decoding_verification_w4a16_amd as w4

    torch = torch_mod()
    q = torch.empty((pk.K, pk.N), dtype=torch.uint8, device=DEV)
    z = torch.empty((pk.K // 128, pk.N), dtype=torch.uint8, device=DEV)
    w4.w4_unpack(pk.qweight_t, pk.zeros_t, pk.N, pk.K, 128, q, z)
    torch.cuda.synchronize()
    return q.cpu().numpy(), z.cpu().numpy()


def diagnostics(y, Y64, A64) -> dict:
    """Contract ratio and the finer GP4 diagnostics."""
    from oracle import check_contract

    ok, worst = check_contract(y, Y64, A64)
    err = np.asarray(y, np.float64) - Y64
    fro = float(np.linalg.norm(err) / max(np.linalg.norm(Y64), 1e-300))
    return {"ok": ok, "worst": worst, "rel_fro": fro, "max_abs": float(np.abs(err).max()) if err.size else 0.0}
