"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with host-only sanitizer instrumentation
(speculative_decoding_verification_w4a16_amd/build_sanitized.py), and the
ABI tests (symbol export, every rejection before a HIP call, the binding's
tensor checks) run against it in a child interpreter with the ASan runtime
preloaded.  Any heap overflow, use after free, misaligned or overflowing
arithmetic in the validation and planning code aborts that run.  Nothing
launches a kernel, so this needs no GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "speculative_decoding_verification_w4a16_amd"))

build_sanitized = pytest.importorskip("build_sanitized")


@pytest.mark.skipif(not os.path.exists(build_sanitized.HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc is not available")
def test_abi_tests_pass_under_asan_and_ubsan():
    lib = build_sanitized.build()
    rt = build_sanitized.runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, W4A16_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the child loads the sanitized library, with the ASan runtime in place
    probe = ("import ctypes, speculative_decoding_verification_w4a16_amd as w; "
             "print(w.LIB_PATH); print(hasattr(ctypes.CDLL(None), '__asan_init'))")
    res = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    assert res.stdout.split() == [lib, "True"], res.stdout
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_binding_checks.py")]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
