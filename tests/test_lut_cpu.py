"""The plan's lookup tables (tile -> tensor for the pack kernels, shard index ->
bucket for the segment walks) checked on the CPU: tests/lut_check.hip compiles
the kernels' own lut_find for the host and compares it with a brute-force scan
at every position of small plans and at the sensitive positions of the
workloads' plans.  A wrong answer there would send a kernel's loads and stores
to the wrong tensor, so this runs before any GPU test."""
import os
import subprocess

import numpy as np
import pytest

from synth import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def lut_prog(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("lut") / "lut_check")
    csrc = os.path.join(ROOT, "gradient_sync_zero_amd", "csrc")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    os.path.join(ROOT, "tests", "lut_check.hip"), os.path.join(csrc, "plan.cpp"),
                    "-o", exe], check=True, capture_output=True)
    return exe


def run(exe, plans):
    text = "".join(f"{P} {align} {cap} {len(numel)} {' '.join(map(str, numel))}\n"
                   for P, align, cap, numel in plans)
    r = subprocess.run([exe], input=text, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
    return r.stdout


def test_lookup_tables_on_workload_plans(lut_prog):
    plans = [(w.world_size, 64, w.bucket_cap_bytes, w.numel)
             for w in (W.by_id(c) for c in (0, 1, 2, 3, 4, 5))]
    out = run(lut_prog, plans)
    assert out.split()[1] == "6"


def test_lookup_tables_on_random_and_edge_plans(lut_prog):
    rng = np.random.default_rng(77)
    plans = []
    for _ in range(60):
        T = int(rng.integers(1, 400))
        numel = [int(x) for x in rng.integers(0, 30000, T)]
        for t in rng.choice(T, size=T // 4, replace=False):
            numel[t] = int(rng.choice([0, 1, 511, 512, 513, 4096]))
        plans.append((int(rng.integers(1, 257)), int(rng.choice([8, 64])),
                      int(rng.integers(1, 200_000)), numel))
    # many one-tile tensors (four starts in every cell), one huge tensor, empty tensors at
    # the ends and around the pack batch boundary at 256, a single bucket
    plans.append((8, 64, 1 << 20, [512] * 3000))
    plans.append((2, 8, 1 << 30, [512] * 200_000 + [3] * 50_000))
    plans.append((8, 64, 1 << 20, [1] * 700 + [0] * 10 + [5000] * 20))
    plans.append((2, 8, 1 << 40, [3, 0, 0, 1 << 26, 0]))
    plans.append((4, 64, 1, [0] * 255 + [700] + [0] * 3 + [1200]))
    plans.append((1, 8, 100, [0] * 300 + [9]))
    out = run(lut_prog, plans)
    assert out.split()[1] == str(len(plans))
