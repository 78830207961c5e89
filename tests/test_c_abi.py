"""CPU: the C ABI from plain C.

tests/host/abi_c.c includes include/kvattn.h as C99 (gcc -pedantic) and
calls the library's host-only entry points from a C program: the supported
K/V pairs and the ones that fail closed, page and workspace sizes (and the
message an invalid geometry leaves), page-table validation, the streaming
planner, one partition-policy step, and null-handle calls.  No GPU work.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "long_context_attention_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_c_program_against_the_header(tmp_path):
    lib = os.path.join(LIBDIR, "libkvattn.so")
    if not os.path.exists(lib):
        pytest.skip("libkvattn.so not built")
    exe = str(tmp_path / "abi_c")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-O1", "-o", exe,
           os.path.join(ROOT, "tests", "host", "abi_c.c"), "-L", LIBDIR, "-lkvattn", f"-Wl,-rpath,{LIBDIR}"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout + run.stderr
