"""bench.py's one-line JSON contract, run for real on a small workload: the
fields the harness reads are present with the right types, the per-call times
add up to the step they were measured in, the roofline fraction is achieved / peak, and the CPU
baseline is the oracle's (the refusal of more than one GPU is a CPU test)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=400):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=timeout, cwd=ROOT)


def test_bench_line_on_the_gpt2_small_share():
    run = run_bench("--config", "1", "--steps", "5", "--warmup", "2", "--no-interleaved")
    assert run.returncode == 0, run.stderr[-2000:]
    lines = [l for l in run.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, run.stdout
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                     ("steps", int), ("warmup", int), ("ms_per_step", float),
                     ("higher_is_better", bool), ("scaling", str), ("dtype", str),
                     ("data", str), ("config", dict), ("roofline", dict),
                     ("cpu_baseline", dict)):
        assert isinstance(d[key], typ), (key, d[key])
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["vs_baseline"] is None and d["data"] == "synthetic" and d["unit"] == "params/s"
    assert d["config"]["workload"] == "gpt2-small-124M-P8" and "model" not in d["config"]
    S = d["config"]["shard_params"]
    assert abs(d["value"] - S / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    k = d["kernels"]
    # the per-call times come from a second pass with events between the calls
    parts = sum(k[n]["ms"] for n in ("shard_reduce_mean", "clip_coef", "shard_adamw_step"))
    with_events = d["step_ms_gpu"]["with_call_events"]["mean"]
    assert parts <= with_events * 1.05, (parts, with_events)
    assert d["step_ms_gpu"]["timed"] <= d["ms_per_step"] * 1.05
    assert d["graph_ms_per_step"] > 0 and d["graph_hbm_frac_of_peak"] > 0
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-12
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]



def test_ddp_bench_line_on_the_gpt2_small_model():
    """The unsharded step's line (--variant ddp): the same contract, its
    kernels' times adding up to at most the step."""
    run = run_bench("--config", "1", "--variant", "ddp", "--steps", "5", "--warmup", "2")
    assert run.returncode == 0, run.stderr[-2000:]
    lines = [l for l in run.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, run.stdout
    d = json.loads(lines[0])
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["unit"] == "params/s"
    assert d["config"]["variant"] == "ddp" and "model" not in d["config"]
    assert abs(d["value"] - d["config"]["total_params"] / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    parts = sum(v["ms"] for v in d["kernels"].values())
    with_events = d["step_ms_gpu"]["with_call_events"]["mean"]
    assert parts <= with_events * 1.05, (parts, with_events)
    assert d["step_ms_gpu"]["timed"] <= d["ms_per_step"] * 1.05
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-12
