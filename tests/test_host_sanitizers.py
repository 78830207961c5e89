"""The library's pure host logic (page-table validation, the streaming
planner with the enqueue sequence the HIP path issues, the adaptive
partition policy) built with AddressSanitizer and UndefinedBehaviorSanitizer
by g++ and run over seeded random configurations (tests/host/host_checks.cpp).
CPU only; no HIP code is compiled here."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_logic_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    src = os.path.join(HERE, "host", "host_checks.cpp")
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-Wall", "-Wextra"]
    build = subprocess.run(["g++", *flags, src, "-o", exe], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    assert "warning" not in build.stderr, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert run.stdout.strip().endswith("ok")
