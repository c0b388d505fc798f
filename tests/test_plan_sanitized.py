"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/plan_fuzz.cpp drives plan.cpp (built with g++ for the host, no device
code) through random and hostile tensor lists, caps, world sizes and granules
and checks each valid plan's invariants; any memory error or undefined
behaviour aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def fuzz_exe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("fuzz") / "plan_fuzz")
    csrc = os.path.join(ROOT, "gradient_sync_zero_amd", "csrc")
    r = subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                        "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", csrc,
                        "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "plan_fuzz.cpp"),
                        os.path.join(csrc, "plan.cpp"), "-o", exe],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("seed", [1, 2])
def test_planner_is_clean_under_sanitizers(fuzz_exe, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzz_exe, str(seed), "1500"], capture_output=True, text=True,
                       timeout=600, env=env)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
    assert int(r.stdout.split()[1]) > 1000          # most draws make a valid plan
