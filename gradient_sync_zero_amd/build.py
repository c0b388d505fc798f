"""Builds libgsz.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LIB = os.path.join(_HERE, "libgsz.so")
# The same sources with the test hooks of include/gsz_test.h compiled in.
TEST_LIB = os.path.join(_HERE, "libgsz_test.so")

# -ffp-contract=off: the AdamW update and the fp32 reduction must keep one
# rounding per operation (no fused multiply-add).  Packed fp32 instructions are
# switched off.  Division and sqrt stay IEEE correctly rounded (clang's HIP
# default); fp32 denormals are kept.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-fno-fast-math",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result",
         "-I", os.path.join(_ROOT, "include"),
         "-Wl,-rpath,/opt/rocm/lib"]
SOURCES = ["csrc/plan.cpp", "csrc/gsz_step.hip"]


def build(verbose: bool = False) -> str:
    """Builds libgsz.so and libgsz_test.so side by side (two hipcc processes)."""
    jobs = []
    for out, extra in ((LIB, []), (TEST_LIB, ["-DGSZ_TEST_HOOKS"])):
        cmd = [HIPCC, *FLAGS, *extra, *SOURCES, "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((out, cmd, subprocess.Popen(cmd, cwd=_HERE)))
    failed = [cmd for _, cmd, proc in jobs if proc.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    for out, _, _ in jobs:
        os.replace(out + ".tmp", out)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
