"""Build a host-sanitizer copy of libw4a16.so: the same sources, with the
host code (the C ABI, its validation and the launch stubs) instrumented by
AddressSanitizer and UndefinedBehaviorSanitizer; device code is built as
usual.  It is for CPU-only runs of the ABI tests (nothing in them launches a
kernel): load it with W4A16_LIB=<path> and LD_PRELOAD=<the ASan runtime>.

Usage: python speculative_decoding_verification_w4a16_amd/build_sanitized.py
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from build import COMMON, HIPCC, SOURCES  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT_DIR = os.path.join(ROOT, "_build", "sanitized")
LIB = os.path.join(OUT_DIR, "libw4a16.so")
# every sanitizer flag applies to the host compilation only
SANITIZE = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime() -> str:
    """The ASan runtime to preload into an uninstrumented interpreter."""
    clang = os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang")
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return out.stdout.strip()


def _digest() -> str:
    h = hashlib.sha256(" ".join(COMMON + SANITIZE).encode())
    csrc = os.path.dirname(SOURCES[0])
    inc = os.path.join(ROOT, "include")
    for d in (csrc, inc):
        for f in sorted(os.listdir(d)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()


def build() -> str:
    """Build (or reuse, when the sources are unchanged) the sanitized library."""
    os.makedirs(OUT_DIR, exist_ok=True)
    stamp = LIB + ".digest"
    dig = _digest()
    if os.path.exists(LIB) and os.path.exists(stamp) and open(stamp).read() == dig:
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *COMMON, *SANITIZE, "-shared", "-o", tmp, *SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building the sanitized libw4a16.so")
    os.replace(tmp, LIB)
    with open(stamp, "w") as fh:
        fh.write(dig)
    return LIB


if __name__ == "__main__":
    print(build())
    print(runtime())
