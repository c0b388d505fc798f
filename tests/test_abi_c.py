"""The boundary is a C ABI: a C11 program that includes include/gsz.h,
links libgsz.so and calls the host-side entry points (planner, plan tables,
hash check, ledger, workspace size, status strings) compiles without a
warning from the header and gives what the Python binding gives.  No device
call is made."""
import os
import shutil
import subprocess

import pytest

import gradient_sync_zero_amd as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SOURCE = r"""
#include <stdio.h>
#include "gsz.h"
#include "gsz_test.h"

int main(void) {
    int64_t numel[5] = {1000, 37, 4096, 0, 5};
    gsz_plan* p = NULL;
    if (gsz_plan_create(numel, 5, 4000, 4, 64, &p) != GSZ_OK) return 1;
    gsz_plan_info info;
    if (gsz_plan_get_info(p, &info) != GSZ_OK) return 2;
    printf("info %d %d %d %lld %lld %llu\n", (int)info.n_tensors, (int)info.n_buckets,
           (int)info.world_size, (long long)info.flat_len, (long long)info.shard_len,
           (unsigned long long)info.hash);
    for (int32_t b = 0; b < info.n_buckets; ++b) {
        gsz_bucket_info bi;
        if (gsz_plan_bucket(p, b, &bi) != GSZ_OK) return 3;
        printf("bucket %d %lld %lld %lld %lld\n", (int)b, (long long)bi.base, (long long)bi.n_elems,
               (long long)bi.chunk, (long long)bi.shard_off);
    }
    for (int32_t t = 0; t < 5; ++t) {
        int64_t off = -1;
        int32_t bkt = -1;
        if (gsz_plan_tensor(p, t, &off, &bkt) != GSZ_OK) return 4;
        printf("tensor %d %lld %d\n", (int)t, (long long)off, (int)bkt);
    }
    size_t dev_bytes = 0;
    if (gsz_plan_device_bytes(p, &dev_bytes) != GSZ_OK) return 7;
    printf("devbytes %zu\n", dev_bytes);
    printf("check_same %d\n", gsz_plan_check(p, info.hash));
    printf("check_other %d %s\n", gsz_plan_check(p, info.hash ^ 1u),
           gsz_status_string(gsz_plan_check(p, info.hash ^ 1u)));
    double bpp = 0.0;
    if (gsz_ledger_bytes_per_param(8, 2, &bpp) != GSZ_OK) return 5;
    size_t ws = 0;
    if (gsz_workspace_bytes(842301952, &ws) != GSZ_OK) return 6;
    printf("ledger %.4f ws %zu\n", bpp, ws);
    printf("bad %d\n", gsz_workspace_bytes(-1, &ws));
    printf("error %s\n", gsz_last_error());
    return gsz_plan_destroy(p);
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_uses_the_abi(tmp_path):
    src = tmp_path / "abi.c"
    src.write_text(C_SOURCE)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(G.LIB_PATH)
    cc = subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
                         "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                         str(src), "-o", str(exe), "-L", libdir, "-lgsz",
                         f"-Wl,-rpath,{libdir}"], capture_output=True, text=True, timeout=120)
    assert cc.returncode == 0, cc.stderr
    assert "gsz.h" not in cc.stderr, cc.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stderr)
    out = {}
    for line in run.stdout.splitlines():
        key, *vals = line.split()
        out.setdefault(key, []).append(vals)

    plan = G.Plan([1000, 37, 4096, 0, 5], 4000, 4)
    n_tensors, n_buckets, P, flat_len, shard_len, h = out["info"][0]
    assert (int(n_tensors), int(n_buckets), int(P)) == (5, plan.n_buckets, 4)
    assert (int(flat_len), int(shard_len), int(h)) == (plan.flat_len, plan.shard_len, plan.hash)
    for b, (idx, base, n, chunk, soff) in enumerate(out["bucket"]):
        bi = plan.bucket(b)
        assert (int(base), int(n), int(chunk), int(soff)) == \
            (bi["base"], bi["n_elems"], bi["chunk"], bi["shard_off"])
    for t, (idx, off, bkt) in enumerate(out["tensor"]):
        assert (int(off), int(bkt)) == plan.tensor(t)
    assert int(out["devbytes"][0][0]) == plan.device_bytes()
    assert out["check_same"][0] == ["0"]
    assert out["check_other"][0][0] == str(G.load().gsz_plan_check(plan.handle, plan.hash ^ 1))
    assert float(out["ledger"][0][0]) == G.ledger_bytes_per_param(8, 2)
    assert int(out["ledger"][0][2]) == G.workspace_bytes(842301952)
    assert int(out["bad"][0][0]) < 0


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_step_client_compiles(tmp_path):
    """tests/c_step_client.c, the C-only client that the GPU tests run through
    the whole step, builds against the header with no warning."""
    from tests.test_gpu_c_client import build_client
    assert os.path.exists(build_client(str(tmp_path)))
