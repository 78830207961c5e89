"""Build the HIP libraries in-tree (gfx950): long_context_attention_amd/libkvattn.so
and the measurement helper libkvattn_probe.so (plain-read ceiling, used by the
benchmark only)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvattn.so")
SOURCES = ["kvattn.hip", "split_kernel.hip", "wide_kernel.hip", "writer_kernel.hip", "copy_kernels.hip", "debug_kernels.hip"]
HEADERS = ["attn_kernels.h", "kernels_common.h", "sched.h"]
PROBE_LIB = os.path.join(HERE, "libkvattn_probe.so")
PROBE_SOURCES = ["read_probe.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off (the compiler would otherwise form them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


def _compile(sources, lib, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = lib + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(os.path.dirname(HERE), "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    errs = "\n".join(l for l in (proc.stderr or "").splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, lib)


def is_stale() -> bool:
    if not os.path.exists(LIB) or not os.path.exists(PROBE_LIB):
        return True
    t = min(os.path.getmtime(LIB), os.path.getmtime(PROBE_LIB))
    deps = [os.path.join(CSRC, f) for f in SOURCES + HEADERS + PROBE_SOURCES]
    deps += [os.path.join(os.path.dirname(HERE), "include", h) for h in ("kvattn.h", "kvattn_probe.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    print(build(verbose=True))
