"""The C ABI is usable from plain C (no GPU needed).

A C99 program that includes include/gqa.h (and the benchmark helper's
include/gqa_bench.h) is compiled with gcc (-Wall
-Werror, strict prototypes), linked against libgqa.so and run: it checks the
version, every status string, the workspace-size functions, and that invalid
calls return their status codes before touching a device.  The header is also
compiled as C++ to check its extern "C" guard.
"""

import os
import shutil
import subprocess

import pytest

import prefill_split_gqa_amd as gqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
LIBDIR = os.path.dirname(gqa.LIB_PATH)

C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "gqa.h"
#include "gqa_bench.h"

static int fails = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL line %d: %s\n", __LINE__, #c); ++fails; } } while (0)

int main(void)
{
    int s;
    void *fake = (void *)0x10000; /* aligned, never dereferenced */
    CHECK(gqa_abi_version() >= 1);
    for (s = GQA_OK; s <= GQA_ERR_SCRATCH; ++s) CHECK(strlen(gqa_status_string(s)) > 0);
    CHECK(gqa_status_string(12345) != NULL);
    CHECK(gqa_decode_workspace_bytes(1, 28, 4, 128, 4096) > ((size_t)16 << 20));
    CHECK(gqa_decode_workspace_bytes(1, 28, 5, 128, 4096) == 0); /* Hq not a multiple of Hkv */
    CHECK(gqa_prefill_workspace_bytes(1, 14, 2, 64, 4097, 4097) >= ((size_t)16 << 20));
    CHECK(gqa_prefill_workspace_bytes(1, 14, 2, 64, 10, 5) == 0); /* Tq > Tk */
    CHECK(gqa_decode_attend(NULL, fake, fake, fake, 1, 28, 4, 128, 10, 10, 0.1f, GQA_F32, fake, 1u << 30, NULL)
          == GQA_ERR_NULL);
    CHECK(gqa_decode_attend(fake, fake, fake, fake, 1, 28, 4, 96, 10, 10, 0.1f, GQA_F32, fake, 1u << 30, NULL)
          == GQA_ERR_UNSUPPORTED);
    CHECK(gqa_prefill_causal(fake, fake, fake, fake, 1, 14, 2, 64, 20, 10, 10, 0.125f, GQA_BF16, fake, 1u << 30,
                             NULL) == GQA_ERR_SHAPE);
    CHECK(gqa_read_probe(fake, 100, fake, NULL) == GQA_ERR_SHAPE);
    printf("c-abi checks: %d failed\n", fails);
    return fails != 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_and_library_from_c99(tmp_path):
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-Wstrict-prototypes", "-I", INC, str(src),
                    "-L", LIBDIR, "-lgqa", "-Wl,-rpath," + LIBDIR, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failed" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_header_compiles_as_cpp(tmp_path):
    src = tmp_path / "abi.cpp"
    src.write_text('#include "gqa.h"\nint main() { return gqa_abi_version() > 0 ? 0 : 1; }\n')
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-fsyntax-only", "-I", INC, str(src)], check=True)
