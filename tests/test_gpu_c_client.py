"""The C ABI used from C alone: tests/c_step_client.c, a C11 program whose
process holds no Python and no torch, runs the ZeRO-1/2 step of every owner
through include/gsz.h and the HIP runtime (its own plan-table buffer,
workspace and device buffers; pack, reduce-mean with the fused norm partials,
clip coefficient, AdamW with the all-gather store).  Its outputs equal the
oracle's on the same seeded inputs: g, master, m, v and the gathered bf16
parameters bit for bit, the norm partials and their total within 1e-12
relative, the clip coefficient and norm exactly."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import gradient_sync_zero_amd as G
from oracle import pack as opack
from oracle.plan import make_plan
from oracle.step import zero_step_all_owners
from synth import workloads as W
from tests import oracle_inputs as OI
from tests.parity import assert_bits

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "tests", "c_step_client.c")


def build_client(out_dir):
    """gcc, C11, against include/gsz.h, libgsz.so and the HIP runtime."""
    exe = os.path.join(out_dir, "c_step_client")
    libdir = os.path.dirname(G.LIB_PATH)
    cc = subprocess.run(["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
                         "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", SOURCE,
                         "-o", exe, "-L", libdir, "-lgsz", "-L", "/opt/rocm/lib", "-lamdhip64",
                         f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib"],
                        capture_output=True, text=True, timeout=120)
    assert cc.returncode == 0, cc.stderr
    assert "warning" not in cc.stderr, cc.stderr
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
@pytest.mark.parametrize("cfg", [0, 5])
def test_c_client_step_equals_oracle(cfg, tmp_path):
    w = W.by_id(cfg)
    P = w.world_size
    exe = build_client(str(tmp_path))
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    grads = [OI.rank_grads(w, q) for q in range(P)]
    for q in range(P):
        np.concatenate(grads[q]).astype(np.uint16).tofile(tmp_path / f"grads_{q}.bin")
    th, m, v = OI.full_state(oplan, w)
    for r in range(P):
        for name, full in (("master", th), ("m", m), ("v", v)):
            opack.owner_view(oplan, full, r).astype(np.float32).tofile(tmp_path / f"{name}_{r}.bin")
    hp = w.hp
    with open(tmp_path / "params.txt", "w") as f:
        f.write(f"{len(w.numel)} {P} {w.bucket_cap_bytes} {hp.lr.hex()} {hp.beta1.hex()} "
                f"{hp.beta2.hex()} {hp.eps.hex()} {hp.weight_decay.hex()} {hp.step} "
                f"{float(hp.max_norm).hex()}\n")
        f.write(" ".join(str(n) for n in w.numel) + "\n")
    print(f"[{w.name}] running the C client", flush=True)
    run = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)

    flats = [opack.pack(oplan, grads[q]) for q in range(P)]
    ref = zero_step_all_owners(oplan, flats, th, m, v, hp)
    S = oplan.shard_len
    for r in range(P):
        g = np.fromfile(tmp_path / f"out_g_{r}.bin", dtype=np.float32)
        assert g.size == S
        assert_bits(g, ref["g"][r], f"C client g owner {r}")
        for key, name in (("theta", "master"), ("m", "m"), ("v", "v")):
            got = np.fromfile(tmp_path / f"out_{name}_{r}.bin", dtype=np.float32)
            assert_bits(got, ref[key][r], f"C client {name} owner {r}")
    gathered = np.fromfile(tmp_path / "out_gathered.bin", dtype=np.uint16)
    assert_bits(gathered, ref["gathered"], "C client gathered bf16")
    parts = np.fromfile(tmp_path / "out_partials.bin", dtype=np.float64)
    for r in range(P):
        assert abs(parts[r] - ref["partials"][r]) <= 1e-12 * ref["partials"][r]
    raw = (tmp_path / "out_clip.bin").read_bytes()
    coef, norm = np.frombuffer(raw[:8], dtype=np.float32)
    total = np.frombuffer(raw[8:], dtype=np.float64)[0]
    assert abs(total - ref["total"]) <= 1e-12 * ref["total"]
    assert norm == ref["norm"] and coef == ref["coef"], (coef, norm, ref["coef"], ref["norm"])
