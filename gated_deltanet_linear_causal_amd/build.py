"""Builds libgdn.so (host C++ + HIP kernels for gfx950) in the package directory, and
libgdn_bench.so (the benchmark's streaming-copy reference kernel).

    python -m gated_deltanet_linear_causal_amd.build

Compiles every time it is called. Packed-fp32 instructions are disabled
(``-target-feature -packed-fp32-ops``); the compiler still vectorises scalar code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_api.cpp", "gdn_kernels.hip", "gdn_verify.hip", "gdn_chunked.hip", "gdn_proj.hip"]
BENCH_LIB = os.path.join(PKG, "libgdn_bench.so")
BENCH_SOURCES = ["bench_copy.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgdn.so)")


def flags(extra=()):
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, *extra]


def build(out: str = LIB, extra=(), verbose: bool = False) -> str:
    """Builds libgdn.so at `out` and the benchmark library beside the package."""
    _build(out, SOURCES, extra, verbose)
    _build(BENCH_LIB, BENCH_SOURCES, extra, verbose)
    return out


def _build(out, sources, extra, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *flags(extra), "-shared", *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("building %s failed" % os.path.basename(out))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
