"""Builds the two generator libraries in-tree (host C with gcc, device HIP for gfx950)."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wl,-rpath,/opt/rocm/lib"]


def _run(cmd):
    subprocess.run(cmd, check=True, cwd=_HERE)


def build(verbose: bool = False) -> None:
    host_out = os.path.join(_HERE, "libsynth_host.so")
    dev_out = os.path.join(_HERE, "libsynth_dev.so")
    cmds = [
        ["gcc", "-O3", "-ffp-contract=off", "-fno-trapping-math", "-fopenmp", "-fPIC", "-shared", "-std=gnu11",
         "philox_host.c", "-o", host_out + ".tmp"],
        [HIPCC, *HIP_FLAGS, "philox_dev.hip", "-o", dev_out + ".tmp"],
    ]
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
    os.replace(host_out + ".tmp", host_out)
    os.replace(dev_out + ".tmp", dev_out)


if __name__ == "__main__":
    build(verbose=True)
