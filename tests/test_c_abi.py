"""The boundary is a C ABI: a C99 program that includes every public header
compiles with -Wall -Wextra -Werror, links against the in-tree libw4a16.so
and runs the calls that need no GPU (byte sizes, launch plans of the linear
and of tree attention, status strings, argument errors returned before any
HIP call).  The same headers
also compile as C++ (-std=c++17)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "speculative_decoding_verification_w4a16_amd")
LIB = os.path.join(PKG, "libw4a16.so")
HEADERS = ("w4a16.h", "w4a16_bench.h", "w4_accept.h", "w4_tree_attn.h", "w4_pass.h")

PROGRAM = r"""
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include "w4a16.h"
#include "w4a16_bench.h"
#include "w4_accept.h"
#include "w4_tree_attn.h"
#include "w4_pass.h"

int main(void) {
    size_t qb = 0, sb = 0, zb = 0;
    /* the Llama-3-70B q projection: the canonical sizes (N % 64 == 0) */
    if (w4_repacked_sizes(8192, 8192, 128, &qb, &sb, &zb) != W4_OK) return 1;
    if (qb != (size_t)8192 * 8192 / 2 || sb != (size_t)8192 * 8192 / 64 || zb != (size_t)8192 * 8192 / 256) return 2;
    /* ragged N pads to whole 64-column chunks */
    if (w4_repacked_sizes(200, 256, 128, &qb, &sb, &zb) != W4_OK || qb != (size_t)256 * 256 / 2) return 3;
    int kernel = -1, splits = -1, kwaves = -1, grid = -1, block = -1, lds = -1;
    if (w4a16_plan(64, 8192, 8192, 128, W4_KERNEL_AUTO, 0, 0, &kernel, &splits, &kwaves, &grid, &block, &lds) != W4_OK)
        return 4;
    if (kernel != W4_KERNEL_MFMA || lds <= 0 || grid < 1 || block < 64 || splits < 1) return 5;
    if (w4a16_plan(1, 8192, 8192, 128, W4_KERNEL_AUTO, 0, 0, &kernel, &splits, &kwaves, &grid, &block, &lds) != W4_OK ||
        kernel != W4_KERNEL_GEMV)
        return 6;
    /* argument errors come back before any HIP call (fake, aligned device addresses) */
    const uint16_t* x = (const uint16_t*)(uintptr_t)0x1000;
    const uint32_t* qt = (const uint32_t*)(uintptr_t)0x2000;
    const uint16_t* st = (const uint16_t*)(uintptr_t)0x3000;
    const uint16_t* zt = (const uint16_t*)(uintptr_t)0x4000;
    float* y = (float*)(uintptr_t)0x100000;
    if (w4a16_linear(x, qt, st, zt, 65, 256, 512, 128, y, NULL) != W4_ERR_UNSUPPORTED) return 7;
    if (w4a16_linear(x, qt, st, zt, 4, 256, 512, 64, y, NULL) != W4_ERR_UNSUPPORTED) return 8;
    if (w4a16_linear(NULL, qt, st, zt, 4, 256, 512, 128, y, NULL) != W4_ERR_INVALID) return 9;
    if (w4a16_linear(x, qt, st, zt, 0, 256, 512, 128, y, NULL) != W4_OK) return 10; /* nothing to do */
    if (strlen(w4_status_str(W4_ERR_INVALID)) == 0 || strlen(w4_status_str(W4_ERR_HIP)) == 0) return 11;
    /* tree attention: the split count and merge a shape uses, host only */
    int tsplits = 0, tmerge = -1;
    if (w4_tree_attention_plan(1, 4096, 64, 8, W4_TREE_MERGE_AUTO, &tsplits, &tmerge) != W4_OK || tsplits < 2 ||
        tmerge != W4_TREE_MERGE_LAUNCH)
        return 12;
    if (w4_tree_attention_plan(1, 512, 64, 8, W4_TREE_MERGE_AUTO, NULL, &tmerge) != W4_OK ||
        tmerge != W4_TREE_MERGE_LAST)
        return 13;
    if (w4_tree_attention_plan(1, 64, 64, 8, 3, NULL, NULL) != W4_ERR_INVALID) return 14;
    if (w4_tree_attention_ex(NULL, NULL, NULL, NULL, NULL, NULL, 0, 0, 64, 8, 128, 0.0f, -1, NULL, NULL) !=
        W4_ERR_INVALID)
        return 15;
    printf("ok %zu %d %d %d\n", qb, splits, grid, block);
    return 0;
}
"""


def _compiler(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} not installed")
    return path


def test_headers_are_c_and_the_library_links_from_c(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("libw4a16.so not built")
    gcc = _compiler("gcc")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-L", PKG, "-lw4a16", f"-Wl,-rpath,{PKG}", "-o", str(exe)], check=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    assert run.stdout.startswith("ok "), run.stdout


def test_headers_compile_as_cpp(tmp_path):
    gxx = _compiler("g++")
    src = tmp_path / "abi.cpp"
    src.write_text("".join(f'#include "{h}"\n' for h in HEADERS) + "int main() { return 0; }\n")
    subprocess.run([gxx, "-std=c++17", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I",
                    os.path.join(ROOT, "include"), str(src)], check=True)
