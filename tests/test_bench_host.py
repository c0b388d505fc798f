"""CPU tests of the benchmark's host logic: one GPU only, and the profile
summaries it writes and reads (synthetic rocprofv3 CSVs in a temporary
directory; the committed profiles are not touched)."""
import csv
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 2
    assert "only --gpus 1" in out.stderr


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_names_template_instances(tmp_path):
    rows = [("void (anonymous namespace)::k_pack<0>(PackPtrs, long const*, int, int, long, long, unsigned short*)",
             4, 2000000, 1000000, 3000000, 8000000),
            ("void (anonymous namespace)::k_pack<2>(PackPtrs, long const*, int, int, long, long, unsigned short*)",
             2, 3000000, 3000000, 3000000, 6000000),
            ("void (anonymous namespace)::k_reduce_mean<8, true, 0, false, true>(RankPtrs, int, float, int, long const*, int, long, long, float*, double*)",
             1, 500, 500, 500, 500)]
    src = tmp_path / "stats.csv"
    _write_csv(src, ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "TotalDurationNs"], rows)
    bench.summarize_trace(str(src), "w", "cmd", out_dir=str(tmp_path))
    text = (tmp_path / "kernel_stats_w.txt").read_text()
    assert "# command: cmd" in text
    lines = [l.split() for l in text.splitlines() if not l.startswith("#")]
    assert lines[0][:3] == ["k_pack", "4", "2000.0"]
    assert lines[1][0] == "k_accumulate"
    assert lines[2][0] == "k_reduce_mean_bf16_wire"


def test_lane_contiguous_reduce_instances_are_named_by_row():
    lc = "void (anonymous namespace)::k_reduce_mean_lc<{}>(RankPtrsT<{}>, int, float, int)"
    assert bench.short_name(lc.format("unsigned short, 8, true, 0, false, false", "unsigned short")) \
        == "k_reduce_mean"
    assert bench.short_name(lc.format("unsigned short, 8, true, 1, false, false", "unsigned short")) \
        == "k_reduce_mean"
    assert bench.short_name(lc.format("unsigned short, 8, true, 2, false, false", "unsigned short")) \
        == "k_reduce_mean_ilv"
    assert bench.short_name(lc.format("float, 8, true, 1, false, false", "float")) \
        == "k_reduce_mean_f32"
    assert bench.short_name(lc.format("unsigned short, 4, true, 0, false, true", "unsigned short")) \
        == "k_reduce_mean_bf16_wire"
    assert bench.short_name(lc.format("unsigned short, 2, false, 0, true, false", "unsigned short")) \
        == "k_allreduce_mean"
    wide = "void (anonymous namespace)::k_reduce_mean<{}>(RankPtrs, int, float, int)"
    assert bench.short_name(wide.format("64, true, 1, false, false")) == "k_reduce_mean"
    assert bench.short_name(wide.format("64, true, 2, false, false")) == "k_reduce_mean_ilv"
    assert bench.short_name(wide.format("0, true, 0, true, false")) == "k_allreduce_mean"
    burst = "void (anonymous namespace)::k_reduce_burst<{}>(RankPtrs, int, float, int)"
    assert bench.short_name(burst.format("64, true, 1, false")) == "k_reduce_burst"
    assert bench.short_name(burst.format("64, true, 0, false")) == "k_reduce_burst"
    assert bench.short_name(burst.format("64, true, 2, false")) == "k_reduce_burst_ilv"
    assert bench.short_name(burst.format("24, true, 1, true")) == "k_reduce_burst_bf16_wire"


def test_bench_names_the_reduce_kernel_the_library_runs():
    """The burst kernel at every world size above 16 on shards of 2^23
    elements or more; the tile kernel below that size; the lane-contiguous
    kernel (named like the tile one) at P <= 16."""
    big = 1 << 23
    assert bench.reduce_kernel(64, 1077760128, "compact") == "k_reduce_burst"
    assert bench.reduce_kernel(64, 1077760128, "interleaved") == "k_reduce_burst_ilv"
    for P in (17, 24, 32, 48, 96, 100, 256):
        assert bench.reduce_kernel(P, big, "flat") == "k_reduce_burst"
        assert bench.reduce_kernel(P, big - 8, "flat") == "k_reduce_mean"
    for P in (2, 8, 16):
        assert bench.reduce_kernel(P, 1 << 30, "compact") == "k_reduce_mean"


def test_counter_summary_scales_by_the_copy_kernel_and_is_keyed(tmp_path):
    # FETCH_SIZE / WRITE_SIZE arrive as several rows per dispatch (one per
    # counter instance); the summary sums them per dispatch, averages per
    # kernel and scales by what the copy kernel of known size read.
    copy = "synth_copy_kernel(u32x4 const*, u32x4*, long)"
    kern = "void (anonymous namespace)::k_adamw<true, false>(float*, float*, float*, float const*, float const*, AdamScalars, long const*, int, long, long, unsigned short*, unsigned short*)"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    copy_bytes = 1 << 20
    fetch = [(1, copy, "FETCH_SIZE", 1024), (1, copy, "FETCH_SIZE", 1024),     # 2048 KiB: x0.5
             (2, kern, "FETCH_SIZE", 3000), (2, kern, "FETCH_SIZE", 1000),
             (3, kern, "FETCH_SIZE", 2000), (3, kern, "FETCH_SIZE", 2000)]
    write = [(1, copy, "WRITE_SIZE", 1024),                                       # 1024 KiB: x1
             (2, kern, "WRITE_SIZE", 700), (3, kern, "WRITE_SIZE", 900)]
    _write_csv(tmp_path / "f.csv", hdr, fetch)
    _write_csv(tmp_path / "w.csv", hdr, write)
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "w", "cmd", copy_bytes,
                        out_dir=str(tmp_path))
    want = 4000 * 1024 * 0.5 + 800 * 1024 * 1.0
    got = bench.read_traffic("k_adamw", "w", profiles_dir=str(tmp_path))
    assert abs(got - want) < 1.0
    assert bench.read_traffic("k_pack", "w", profiles_dir=str(tmp_path)) is None
    # a summary taken on other kernel sources is not used
    p = tmp_path / "traffic_w.txt"
    p.write_text(p.read_text().replace(bench.kernel_source_digest(), "0" * 64))
    assert bench.read_traffic("k_adamw", "w", profiles_dir=str(tmp_path)) is None


def test_committed_profiles_record_the_command_that_made_them():
    prof = os.path.join(ROOT, "profiles")
    names = sorted(n for n in os.listdir(prof) if n.endswith(".txt"))
    assert names
    for n in names:
        cmd = [l for l in open(os.path.join(prof, n)) if l.startswith("# command:")]
        assert len(cmd) == 1, n
        text = cmd[0][len("# command:"):].strip()
        assert text.startswith("rocprofv3 ") and "-- python3 bench.py --config" in text, (n, text)


def test_profile_commands_match_the_summary_kinds():
    c = bench.profile_commands(3, "t", "f", "w")
    assert "--kernel-trace --stats" in c["trace"] and "--pmc" not in c["trace"]
    assert "--pmc FETCH_SIZE" in c["fetch"] and "--pmc WRITE_SIZE" in c["write"]
    assert "-d t " in c["trace"] and "-d f " in c["fetch"] and "-d w " in c["write"]
    assert all("--config 3" in v for v in c.values())
    assert bench._raw_dir(os.path.join(ROOT, "x", "y", "k.csv")) == os.path.join("x", "y")
    d = bench.profile_commands(2, "t", "f", "w", variant="ddp")
    assert all("--config 2 --variant ddp" in v for v in d.values())
    assert bench.profile_name("gpt-1.3B-P8", "ddp") == "gpt-1.3B-P8-ddp"
    assert bench.profile_name("gpt-1.3B-P8", "zero") == "gpt-1.3B-P8"


def test_counter_summary_of_any_counters(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = [(1, "void (anonymous namespace)::k_adamw<false, true>(float*)", "A_sum", 10.0),
            (1, "void (anonymous namespace)::k_adamw<false, true>(float*)", "B_sum", 1.0),
            (1, "void (anonymous namespace)::k_adamw<false, true>(float*)", "B_sum", 2.0),
            (2, "void (anonymous namespace)::k_adamw<false, true>(float*)", "A_sum", 30.0),
            (2, "void (anonymous namespace)::k_adamw<false, true>(float*)", "B_sum", 5.0),
            (3, "synth_fill_kernel(int)", "A_sum", 99.0)]
    src = tmp_path / "c.csv"
    _write_csv(src, hdr, rows)
    bench.summarize_counters(str(src), "w", "rocprofv3 --pmc A_sum B_sum -- python3 bench.py --config 3",
                             "ab", out_dir=str(tmp_path))
    text = (tmp_path / "counters_ab_w.txt").read_text()
    body = [l.split() for l in text.splitlines() if not l.startswith("#")]
    assert body == [["k_adamw", "2", "2.0000e+01", "4.0000e+00"]]   # per-dispatch sums, then means


def test_benchmark_and_package_import_nothing_from_tests():
    """bench.py assembles its inputs with synth/placement.py; neither it nor
    the product package may depend on the test package."""
    import ast
    files = [os.path.join(ROOT, "bench.py")]
    for d in ("gradient_sync_zero_amd", "synth"):
        files += [os.path.join(ROOT, d, f) for f in os.listdir(os.path.join(ROOT, d))
                  if f.endswith(".py")]
    for path in files:
        tree = ast.parse(open(path).read())
        for node in ast.walk(tree):
            names = []
            if isinstance(node, ast.Import):
                names = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                names = [node.module or ""]
            assert not any(n == "tests" or n.startswith("tests.") for n in names), (path, names)


def test_cpu_baseline_sample_is_the_workloads_own_inputs():
    """The oracle baseline's window holds exactly the values the oracle's own
    placement gives the first n shard elements (all ranks and the state)."""
    import numpy as np
    from oracle.plan import make_plan
    from synth import workloads as W
    from tests import oracle_inputs as OI
    w = W.by_id(1)
    n, contribs, state = bench._oracle_sample(w, 2, 300_000)
    plan = make_plan(w.numel, w.bucket_cap_bytes, w.world_size)
    idx = OI.shard_param_index(plan, 2)[:n]
    assert n == 300_000 and len(contribs) == w.world_size
    for q in (0, 5, 7):
        assert np.array_equal(contribs[q], OI.values_at(w, W.KIND_GRAD, q, w.grad_std, 2, idx))
    for (kind, std, mode), arr in zip(OI.STATE_KINDS, state):
        assert np.array_equal(arr.view(np.uint32), OI.values_at(w, kind, 0, std, mode, idx).view(np.uint32))


def test_product_path_never_reaches_the_oracle():
    """The oracle is test infrastructure: the product package and the input
    placement import nothing from it, and bench.py only inside its CPU
    baseline (_oracle_sample and cpu_baseline)."""
    import ast
    files = []
    for d in ("gradient_sync_zero_amd", "synth"):
        files += [os.path.join(ROOT, d, f) for f in os.listdir(os.path.join(ROOT, d))
                  if f.endswith(".py")]
    for path in files:
        for node in ast.walk(ast.parse(open(path).read())):
            names = []
            if isinstance(node, ast.Import):
                names = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                names = [node.module or ""]
            assert not any(n == "oracle" or n.startswith("oracle.") for n in names), (path, names)
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    allowed = {"_oracle_sample", "cpu_baseline"}
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef) and fn.name not in allowed:
            for node in ast.walk(fn):
                if isinstance(node, ast.ImportFrom) and (node.module or "").startswith("oracle"):
                    raise AssertionError(f"bench.py: {fn.name} imports {node.module}")
    for node in tree.body:                       # nothing at module level either
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
            assert not any(m.startswith("oracle") for m in mods), mods
