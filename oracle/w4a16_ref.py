"""Plain float64 CPU oracle of the W4A16 verify linear.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg do.  It shares no code with the HIP library.

What it computes, and where that comes from:

* "Speculative Decoding Meets Quantization" (menfem.com knowledge-base note,
  section "Abstract"; the same abstract on the shd-paper.top summary of
  arXiv 2505.22179, section "摘要（原文）"): the target model's weights are
  quantised to 4 bits while activations stay 16-bit, and verification runs
  the target's matrix multiplications over several draft tokens in one
  forward pass.  The ordoresearch.ai review (sections "Research Landscape"
  and "Limitations Worth Noting") adds that the study is weight-only.
* The pages give no formula, group size or packing.  The plainest reading
  of a weight-only 4-bit linear with asymmetric group quantisation is

      y[m, n] = sum_k x[m, k] * (q[k, n] - z[k // g, n]) * s[k // g, n]

  with x bf16, q and z unsigned 4-bit codes, s an fp16 scale per
  (group, column), g = 128, and fp32 output.  The oracle evaluates it
  exactly in float64: every dequantised weight (q - z) * s and every
  product with a bf16 x is exact in float64, so the only rounding is in the
  float64 sum.
* Verification of M draft tokens is M rows of x through the same weights
  (ordoresearch.ai review, "Research Landscape": the target checks the
  drafted tokens in one batched forward pass).  The oracle evaluates rows
  one at a time with one routine, so verifying M tokens is, bit for bit, M
  single-token passes.

Canonical packed input format (see ``synth``): qweight int32 [K/8, N] packed
along K (nibble i of word (j, n) is q[8j+i, n]); scales uint16 fp16 bits
[K/g, N]; zeros int32 [K/g, N/8] packed along N (nibble i of word (G, j) is
z[G, 8j+i]); x uint16 bf16 bits [M, K]; words are read as uint32.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
something other than itself (brute-force exact sums, closed forms, one-hot
probes, integer GEMMs and the hand-worked fixture in ``tests/golden``).
"""
from __future__ import annotations

import numpy as np

#: Contract: |y - Y64| <= CONTRACT_RTOL * sum_k |x_k w_k| per element.
CONTRACT_RTOL = 4e-3


def unpack_qweight(qweight: np.ndarray) -> np.ndarray:
    """O1: qweight int32 [K/8, N] -> codes uint8 [K, N]; q[8j+i, n] = (word >> 4i) & 15."""
    w = np.ascontiguousarray(qweight).view(np.uint32)
    kw, n = w.shape
    out = np.empty((kw, 8, n), np.uint8)
    for i in range(8):
        out[:, i, :] = (w >> np.uint32(4 * i)) & np.uint32(0xF)
    return out.reshape(kw * 8, n)


def unpack_zeros(zeros: np.ndarray) -> np.ndarray:
    """O2: zeros int32 [K/g, N/8] -> zero points uint8 [K/g, N]; z[G, 8j+i] = (word >> 4i) & 15."""
    w = np.ascontiguousarray(zeros).view(np.uint32)
    ng, nw = w.shape
    out = np.empty((ng, nw, 8), np.uint8)
    for i in range(8):
        out[:, :, i] = (w >> np.uint32(4 * i)) & np.uint32(0xF)
    return out.reshape(ng, nw * 8)


def scales_to_f64(scales: np.ndarray) -> np.ndarray:
    """O3: fp16 bit patterns -> float64 (exact: every fp16 value is a float64)."""
    return np.ascontiguousarray(scales).view(np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(x_bits: np.ndarray) -> np.ndarray:
    """O5: bf16 bit patterns -> float64 (exact: bf16 is the top half of an fp32)."""
    u = np.ascontiguousarray(x_bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def dequant64(q: np.ndarray, z: np.ndarray, s64: np.ndarray, group: int) -> np.ndarray:
    """O4: W64[k, n] = (q[k, n] - z[k // g, n]) * s[k // g, n] in float64 (exact)."""
    K, N = q.shape
    G = K // group
    d = q.astype(np.int16).reshape(G, group, N) - z.astype(np.int16).reshape(G, 1, N)
    return (d.astype(np.float64) * s64.reshape(G, 1, N)).reshape(K, N)


def _weights64(qweight, scales, zeros, group, n0=0, n1=None):
    if n1 is None:
        n1 = np.asarray(qweight).shape[1]
    if n0 % 8 or n1 % 8:
        raise ValueError("column slice must be 8-aligned")
    q = unpack_qweight(np.asarray(qweight)[:, n0:n1])
    z = unpack_zeros(np.asarray(zeros)[:, n0 // 8:n1 // 8])
    s = scales_to_f64(np.asarray(scales)[:, n0:n1])
    return dequant64(q, z, s, group)


def linear64(x_bits, qweight, scales, zeros, group: int = 128):
    """O6: (Y64, A64) with Y64 = X64 @ W64 and A64 = |X64| @ |W64|, float64 [M, N].

    Rows are evaluated one at a time with the same routine, so the result for
    row m does not depend on how many other rows are verified with it."""
    W64 = _weights64(qweight, scales, zeros, group)
    return _rows(x_bits, W64)


def linear64_columns(x_bits, qweight, scales, zeros, group: int, n0: int, n1: int):
    """O6 restricted to output columns [n0, n1) (8-aligned); same arithmetic per element."""
    W64 = _weights64(qweight, scales, zeros, group, n0, n1)
    return _rows(x_bits, W64)


def linear64_gemm(x_bits, qweight, scales, zeros, group: int, n0: int, n1: int):
    """O6 over output columns [n0, n1) (8-aligned) as two matrix products,
    Y64 = X64 @ W64 and A64 = |X64| @ |W64| (float64 BLAS), for checks at full
    width where the row-by-row form would read every weight once per row.
    The same definition as ``linear64``; only the float64 summation order
    differs (within K * 2**-52 * A64 of it, pinned in tests)."""
    W64 = _weights64(qweight, scales, zeros, group, n0, n1)
    X64 = bf16_bits_to_f64(np.atleast_2d(x_bits))
    return X64 @ W64, np.abs(X64) @ np.abs(W64)


def _rows(x_bits, W64):
    X64 = bf16_bits_to_f64(np.atleast_2d(x_bits))
    M = X64.shape[0]
    N = W64.shape[1]
    Y = np.empty((M, N), np.float64)
    A = np.empty((M, N), np.float64)
    absW = np.abs(W64)
    for m in range(M):
        Y[m] = X64[m] @ W64
        A[m] = np.abs(X64[m]) @ absW
    return Y, A


def check_contract(y, Y64, A64, rtol: float = CONTRACT_RTOL):
    """O7: returns (ok, worst) where worst = max |y - Y64| / (rtol * A64) (0/0 -> 0).

    The contract is |y - Y64| <= rtol * A64 for every element; where A64 == 0
    the element must be exactly 0."""
    y = np.asarray(y, np.float64)
    err = np.abs(y - Y64)
    bound = rtol * A64
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    return bool(worst <= 1.0), worst


def round_to_bf16(v) -> np.ndarray:
    """bf16 epilogue (an output-type option; the pages leave the output type
    open): the bf16 value nearest to each finite float32 input, ties to the
    even significand, as uint16 bit patterns.  Written from the definition:
    the two bf16 neighbours of v are its truncation toward zero and the next
    bf16 away from zero; the nearer wins, measured exactly in float64."""
    a = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("finite inputs only")
    u = a.view(np.uint32).astype(np.uint64)
    lo = u & np.uint64(0xFFFF0000)                 # toward zero
    hi = lo + np.uint64(0x00010000)                # away from zero (may carry into the exponent: still correct)
    vlo = lo.astype(np.uint32).view(np.float32).astype(np.float64)
    vhi = hi.astype(np.uint32).view(np.float32).astype(np.float64)
    # past the largest bf16 the next step is the overflow threshold 2^128
    vhi = np.where(np.isinf(vhi), np.sign(vhi) * 2.0 ** 128, vhi)
    x = a.astype(np.float64)
    dlo, dhi = np.abs(x - vlo), np.abs(vhi - x)
    lo_even = ((lo >> np.uint64(16)) & np.uint64(1)) == 0
    take_hi = (dhi < dlo) | ((dhi == dlo) & ~lo_even)
    return np.where(take_hi, hi, lo).astype(np.uint64) >> np.uint64(16)

