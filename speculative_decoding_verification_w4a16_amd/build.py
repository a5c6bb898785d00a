"""Build libw4a16.so (the HIP library) in-tree for gfx950 with hipcc.

Usage: python speculative_decoding_verification_w4a16_amd/build.py [--asm]
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4a16.so")
SOURCES = [os.path.join(CSRC, f) for f in ("w4a16_kernels.hip", "w4_pass.hip", "w4_accept.hip", "w4_tree_attn.hip",
                                          "w4a16_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-FP32 VALU forms are disabled for all device code (the compiler would
# otherwise form v_pk_{add,mul,fma}_f32 from scalar float code).  MFMA
# accumulators are kept in architectural VGPRs: with a one-wave-per-SIMD
# register budget the compiler otherwise places them in AGPRs, which costs a
# v_accvgpr_read per epilogue operand and slows independent MFMA chains.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form", "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *COMMON, "-shared", "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libw4a16.so")
    os.replace(tmp, LIB)
    return LIB


def dump_asm(out_path: str) -> None:
    """Device assembly of the kernels (for reading register use and waitcnts)."""
    cmd = [HIPCC, *COMMON, "-S", "--cuda-device-only", "-o", out_path, SOURCES[0]]
    subprocess.run(cmd, check=True, capture_output=True)


if __name__ == "__main__":
    path = build(verbose=True)
    print(path)
    if "--asm" in sys.argv:
        out_dir = os.path.join(os.path.dirname(HERE), "_build")
        os.makedirs(out_dir, exist_ok=True)
        dump_asm(os.path.join(out_dir, "w4a16_kernels.s"))
