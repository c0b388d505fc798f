#!/usr/bin/env python3
"""Benchmark of one rank's share of a synchronous data-parallel step on one
MI355X.  The timed step is the metric's: ring-order reduce-mean of the P
ranks' contributions (with the fused squared-norm partial) -> clip
coefficient -> AdamW on the owned shard (fp32 master/m/v in place, bf16
parameters out), (2P + 34) bytes per shard element.  The bucket pack, the
first part of a rank's share, is timed as its own row.

Workload (default, --config 4): the 70B Llama-shaped share -- 68,976,648,192
parameters in 723 tensors, P = 64 simulated ranks, 25 MiB buckets, owner 0's
shard of 1,077,760,128 elements, its 64 shard-compact contributions (138 GB)
resident in HBM with the fp32 state.  --config 2 and 3 (the 1.3B model and
the 7B share, P = 8) reduce over the ranks' whole bucket-flat buffers and
write the all-gather layout.

Prints one JSON line (see the fields below).  Only N = 1 is supported: the
simulated ranks live on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("params/s and achieved HBM GB/s (% of peak) for reduce-mean + AdamW shard step")
HBM_PEAK_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="turn a rocprofv3 kernel_stats.csv into profiles/kernel_stats_<workload>.txt")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) into profiles/traffic_<workload>.txt")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("CSV", "TAG"),
                    help="turn a rocprofv3 counter_collection.csv with any counters into "
                         "profiles/counters_<TAG>_<workload>.txt")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 50 for the workloads up to 1.3B, 20 for the "
                         "7B and 70B shares)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4,
                    help="workload id (synth.workloads); default 4, the 70B share (P = 64)")
    ap.add_argument("--layout", choices=["auto", "flat", "compact", "interleaved"], default="auto",
                    help="contributions: bucket-flat (the P ranks' whole flat buffers), "
                         "shard-compact (P buffers of S elements) or one rank-interleaved "
                         "receive buffer; auto = flat when it fits (up to the 7B share), else "
                         "compact")
    ap.add_argument("--no-interleaved", action="store_true",
                    help="skip the second pass over a rank-interleaved receive buffer")
    ap.add_argument("--owner", type=int, default=0)
    ap.add_argument("--variant", choices=["zero", "ddp"], default="zero",
                    help="zero: the ZeRO-1/2 shard step (default); ddp: the unsharded step "
                         "(all-reduce, replicated AdamW, unpack)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the step captured as one HIP graph (graph_ms_per_step)")
    ap.add_argument("--copy-gib", type=float, default=4.0,
                    help="size of the plain copy used as the measured HBM ceiling")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 50 if args.config <= 2 else 20
    return args


def ensure_built():
    need = [os.path.join(ROOT, "gradient_sync_zero_amd", "libgsz.so"),
            os.path.join(ROOT, "synth", "libsynth_dev.so"),
            os.path.join(ROOT, "synth", "libsynth_host.so")]
    if not all(os.path.exists(p) for p in need):
        import __graft_entry__
        __graft_entry__.build()


SHORT = {"k_pack": "k_pack", "k_reduce_mean": "k_reduce_mean", "k_adamw": "k_adamw",
         "k_clip": "k_clip", "k_finalize": "k_finalize", "k_zero_pads": "k_zero_pads",
         "synth_copy_kernel": "copy", "synth_fill_kernel": "synth_fill", "k_ag_write": "k_ag_write",
         "k_sqnorm": "k_sqnorm", "synth_read_streams_kernel": "read_streams_probe",
         "synth_read_kernel": "read_probe", "synth_write_kernel": "write_probe"}


def reduce_kernel(P, S, layout):
    """Short name of the kernel the library runs for a bf16 shard reduce (fp32
    on the wire): at P > 16 the burst kernel on shards of 2^23 elements or
    more, else the one-tile-per-block kernel; the lane-contiguous kernel
    (named like the tile one) at P <= 16."""
    base = "k_reduce_burst" if P > 16 and S >= 1 << 23 else "k_reduce_mean"
    return base + ("_ilv" if layout == "interleaved" else "")


def short_name(full):
    # template instances that move different bytes get their own names
    if "k_pack<1>" in full:
        return "k_unpack"
    if "k_pack<2>" in full:
        return "k_accumulate"
    if "k_reduce_burst<" in full:            # <PS, NORM, LAY, W16>
        args = [a.strip() for a in full.split("k_reduce_burst<")[1].split(">")[0].split(",")]
        if len(args) == 4 and args[3] == "true":
            return "k_reduce_burst_bf16_wire"
        if len(args) >= 3 and args[2] == "2":
            return "k_reduce_burst_ilv"
        return "k_reduce_burst"
    if "k_reduce_mean<" in full:             # <PS, NORM, LAY, OUTFLAT, W16>
        args = [a.strip() for a in full.split("k_reduce_mean<")[1].split(">")[0].split(",")]
        if len(args) == 5 and args[4] == "true":
            return "k_reduce_mean_bf16_wire"
        if len(args) >= 4 and args[3] == "true":
            return "k_allreduce_mean"
        if len(args) >= 3 and args[2] == "2":
            return "k_reduce_mean_ilv"
    if "k_reduce_mean_lc<" in full:          # <T, PS, NORM, LAY, OUTFLAT, W16>
        args = [a.strip() for a in full.split("k_reduce_mean_lc<")[1].split(">")[0].split(",")]
        if args[0] == "float":
            return "k_reduce_mean_f32"
        if len(args) == 6 and args[5] == "true":
            return "k_reduce_mean_bf16_wire"
        if len(args) == 6 and args[4] == "true":
            return "k_allreduce_mean"
        if len(args) >= 4 and args[3] == "2":
            return "k_reduce_mean_ilv"
        return "k_reduce_mean"
    if "k_finalize_ranges" in full:
        return "k_finalize_ranges"
    if "k_pack_f32<false>" in full:
        return "k_pack_f32"
    if "k_pack_f32<true>" in full:
        return "k_accumulate_f32"
    if "k_reduce_mean_f32" in full:
        return "k_reduce_mean_f32"
    if "k_zero_pads_f32" in full:
        return "k_zero_pads_f32"
    for k, v in SHORT.items():
        if k in full:
            return v
    if "FillFunctor" in full:
        return "torch_fill"
    if "rocclr" in full:
        return "hip_runtime_copy"
    name = full.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0].split("<")[0][-40:]


def gpu_step_stats(ev):
    """Mean, median and min over the timed steps of the GPU time from each
    step's first event to its last."""
    import numpy as np
    t = [e[0].elapsed_time(e[-1]) for e in ev]
    return dict(mean=float(np.mean(t)), median=float(np.median(t)), min=float(np.min(t)))


def timed_steps(step, names, steps):
    """Times `steps` steps back to back, with one event before the first and one
    after the last: an event recorded between the calls of a step costs it
    10-16 us (measured on the 1.3B model and the 7B share), so the per-call
    breakdown comes from a second pass of as many steps with events between the
    calls.  Returns (wall ms per step, GPU ms per step, per-call samples in ms,
    per-step GPU stats of the second pass)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_wall = (time.perf_counter() - t0) / steps * 1e3
    ms_gpu = e0.elapsed_time(e1) / steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
          for _ in range(steps)]
    for k in range(steps):
        step(ev[k])
    torch.cuda.synchronize()
    samples = {n: [ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(steps)]
               for i, n in enumerate(names)}
    return ms_wall, ms_gpu, samples, gpu_step_stats(ev)


def graph_steps(step, warmup, steps):
    """The same step captured once into a HIP graph and replayed `steps` times:
    wall ms per replay.  The launch gaps between the calls shrink."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def profile_commands(config, trace_dir, fetch_dir, write_dir, variant="zero", layout="auto"):
    """The rocprofv3 command lines (run from the repository root) whose output
    the summaries below are made from: a kernel trace of the default bench of
    a workload, and one counter pass each for FETCH_SIZE and WRITE_SIZE, each
    writing <dir>/bench_*.csv."""
    var = " --variant ddp" if variant == "ddp" else ""
    if layout != "auto":
        var += f" --layout {layout}"
    bench_args = f"python3 bench.py --config {config}{var} --no-cpu-baseline"
    short = f"python3 bench.py --config {config}{var} --steps 3 --warmup 1 --no-cpu-baseline"
    return {"trace": f"rocprofv3 --kernel-trace --stats -f csv -d {trace_dir} "
                     f"-o bench -- {bench_args}",
            "fetch": f"rocprofv3 --pmc FETCH_SIZE -f csv -d {fetch_dir} -o bench -- {short}",
            "write": f"rocprofv3 --pmc WRITE_SIZE -f csv -d {write_dir} -o bench -- {short}"}


def profile_name(workload, variant, layout="auto"):
    """Name of a workload's profile summaries: the unsharded (DDP) step and
    the rank-interleaved receive layout get their own files."""
    name = f"{workload}-ddp" if variant == "ddp" else workload
    return f"{name}-interleaved" if layout == "interleaved" else name


def _raw_dir(csv_path):
    """The -d directory of the rocprofv3 run that wrote csv_path, relative to
    the repository root when it lies inside it."""
    d = os.path.dirname(os.path.abspath(csv_path))
    rel = os.path.relpath(d, ROOT)
    return d if rel.startswith("..") else rel


def summarize_trace(csv_path, workload, command, out_dir=None):
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    out = [f"# rocprofv3 kernel statistics: {workload}", "#", f"# command: {command}", "#",
           f"# {'kernel':<16} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_ms':>10}"]
    for r in rows:
        out.append(f"  {short_name(r['Name']):<16} {int(r['Calls']):>6} "
                   f"{float(r['AverageNs']) / 1e3:>10.1f} {float(r['MinNs']) / 1e3:>10.1f} "
                   f"{float(r['MaxNs']) / 1e3:>10.1f} {float(r['TotalDurationNs']) / 1e6:>10.2f}")
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"kernel_stats_{workload}.txt")
    open(path, "w").write("\n".join(out) + "\n")
    print(path)


def _pmc_per_dispatch(csv_path, counter):
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if r.get("Counter_Name") != counter:
            continue
        d = r["Dispatch_Id"]
        name = short_name(r["Kernel_Name"])
        per.setdefault(d, [name, 0.0])
        per[d][1] += float(r["Counter_Value"])
    by = {}
    for name, v in per.values():
        by.setdefault(name, []).append(v)
    return by


KERNEL_SOURCES = ("gsz_device.h", "gsz_internal.h", "gsz_kernels_adamw.h", "gsz_kernels_pack.h",
                  "gsz_kernels_reduce.h", "gsz_step.hip")


def _code_tokens(text):
    """C++ source without its comments, whitespace runs collapsed: what a
    comment-only edit leaves unchanged.  String literals are kept whole."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_digest():
    """SHA-256 over the library's kernel sources (names and code, comments and
    whitespace left out), the key that ties a counter summary to the kernels it
    measured."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(name.encode() + b"\0")
        text = open(os.path.join(ROOT, "gradient_sync_zero_amd", "csrc", name)).read()
        h.update(_code_tokens(text).encode())
    return h.hexdigest()


def summarize_pmc(fetch_csv, write_csv, workload, command, copy_bytes, out_dir=None):
    """FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by the ratio
    of known bytes to what it reads for the plain copy of copy_bytes."""
    import numpy as np
    f = _pmc_per_dispatch(fetch_csv, "FETCH_SIZE")
    w = _pmc_per_dispatch(write_csv, "WRITE_SIZE")
    cf = float(np.median(f["copy"])) * 1024
    cw = float(np.median(w["copy"])) * 1024
    sf, sw = copy_bytes / cf, copy_bytes / cw
    digest = kernel_source_digest()
    out = [f"# HBM traffic per launch from rocprofv3 counters: {workload}", "#",
           f"# command: {command}", "#",
           f"# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by the copy kernel's",
           f"# known bytes ({copy_bytes} read, {copy_bytes} written): fetch x {sf:.4f}, "
           f"write x {sw:.4f}.", "# A kernel edited after this file was written gets traffic = null.",
           f"source_sha256 = {digest}",
           f"copy.fetch_scale = {sf:.6f}", f"copy.write_scale = {sw:.6f}"]
    for name in sorted(set(f) & set(w)):
        if name in ("synth_fill", "torch_fill", "hip_runtime_copy"):
            continue
        fb = float(np.mean(f[name])) * 1024 * sf
        wb = float(np.mean(w[name])) * 1024 * sw
        out += [f"{name}.launches = {len(f[name])}",
                f"{name}.fetch_bytes_per_launch = {fb:.0f}",
                f"{name}.write_bytes_per_launch = {wb:.0f}",
                f"{name}.hbm_bytes_per_launch = {fb + wb:.0f}"]
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"traffic_{workload}.txt")
    open(path, "w").write("\n".join(out) + "\n")
    print(path)


def summarize_counters(csv_path, workload, command, tag, out_dir=None):
    """Per-kernel mean per dispatch of every counter in one rocprofv3 counter
    CSV (any counters), written to profiles/counters_<tag>_<workload>.txt."""
    import numpy as np
    names = sorted({r["Counter_Name"] for r in __import__("csv").DictReader(open(csv_path))})
    by = {n: _pmc_per_dispatch(csv_path, n) for n in names}
    kernels = sorted({k for n in names for k in by[n]} - {"synth_fill", "torch_fill",
                                                          "hip_runtime_copy"})
    out = [f"# rocprofv3 counters per dispatch (mean over dispatches): {workload}", "#",
           f"# command: {command}", "#",
           f"# kernel sources (as for the traffic summaries): source_sha256 = {kernel_source_digest()}",
           "#",
           "# " + f"{'kernel':<24} {'dispatches':>10} " + " ".join(f"{n:>32}" for n in names)]
    for k in kernels:
        n_disp = max(len(by[n].get(k, [])) for n in names)
        vals = " ".join(f"{float(np.mean(by[n][k])):>32.4e}" if k in by[n] else f"{'-':>32}"
                        for n in names)
        out.append(f"  {k:<24} {n_disp:>10} {vals}")
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"counters_{tag}_{workload}.txt")
    open(path, "w").write("\n".join(out) + "\n")
    print(path)


def read_traffic(kernel, workload, profiles_dir=None):
    """HBM bytes per launch from the committed counter summary, or None if it
    is missing or was taken on a different kernel source."""
    path = os.path.join(profiles_dir or os.path.join(ROOT, "profiles"), f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^\s*([\w.]+)\s*=\s*(\S+)\s*$", line)
        if m:
            kv[m.group(1)] = m.group(2)
    digest = kernel_source_digest()
    if kv.get("source_sha256") != digest:
        return None
    key = f"{kernel}.hbm_bytes_per_launch"
    return float(kv[key]) if key in kv else None


def _oracle_sample(w, owner, n_max):
    """Host inputs of the oracle baseline: the first n shard elements of the
    owner's shard (n <= n_max), placed with the oracle's plan: the P ranks'
    bf16 contributions for those elements and the owner's fp32 master, m, v
    (pads zero), from the same seeded generator as the device inputs."""
    import numpy as np
    from oracle.plan import make_plan
    from synth import gen
    from synth import workloads as W

    plan = make_plan(w.numel, w.bucket_cap_bytes, w.world_size)
    n = min(plan.shard_len, n_max)
    pre = np.cumsum([0] + list(w.numel))
    pieces = []          # (shard offset, parameter index, length) inside [0, n)
    for b, bk in enumerate(plan.buckets):
        if bk.shard_off >= n:
            break
        cs, ce = plan.chunk_range(b, owner)
        for t in bk.tensors:
            ts, te = plan.tensor_offset[t], plan.tensor_offset[t] + plan.numel[t]
            lo, hi = max(cs, ts), min(ce, te)
            so = bk.shard_off + (lo - cs)
            if lo < hi and so < n:
                pieces.append((so, int(pre[t]) + (lo - ts), min(hi - lo, n - so)))

    def fill(kind, rank, std, mode):
        out = np.zeros(n, dtype=np.uint16 if mode == gen.MODE_BF16 else np.float32)
        for so, pi, ln in pieces:
            gen.host_fill(w.cfg_id, kind, rank, pi, ln, std, mode, out=out[so:so + ln])
        return out

    contribs = [fill(W.KIND_GRAD, q, w.grad_std, gen.MODE_BF16) for q in range(w.world_size)]
    state = [fill(kind, 0, std, mode) for kind, std, mode in
             ((W.KIND_MASTER, W.MASTER_STD, gen.MODE_F32), (W.KIND_EXP_AVG, W.EXP_AVG_STD, gen.MODE_F32),
              (W.KIND_EXP_AVG_SQ, W.EXP_AVG_SQ_STD, gen.MODE_ABS))]
    return n, contribs, state


def cpu_baseline(w, owner, seconds=10.0):
    """The oracle as it stands, timed on the host over a window of the same
    workload: the first ~2^28 / P elements of the owner's shard (the P ranks'
    contributions for them, 512 MiB in all) through the metric's step --
    ring-order reduce-mean, squared-norm partial, clip coefficient (the other
    ranks' partials stand in as copies of this one, as on the GPU) and AdamW
    with the bf16 result.  Timed twice: on one core, and with the window cut
    into one slice per host core, each slice run by a thread through the same
    oracle functions (NumPy releases the interpreter lock inside its array
    operations).  Input generation is not timed."""
    import concurrent.futures as cf

    import numpy as np
    from oracle.adamw import adamw
    from oracle.norm import clip_coef, sqnorm_partial, total
    from oracle.reduce import reduce_mean

    P = w.world_size
    hp = w.hp
    log(f"[cpu] generating the oracle sample: {P} contributions of up to {(1 << 28) // P} elements")
    n, contribs, (th0, m0, v0) = _oracle_sample(w, owner, (1 << 28) // P)
    cores = max(1, min(16, os.cpu_count() or 1))

    def step(lo, hi):
        g = reduce_mean([c[lo:hi] for c in contribs], owner)
        return g, sqnorm_partial(g)

    def update(g, lo, hi, coef):
        return adamw(th0[lo:hi], m0[lo:hi], v0[lo:hi], g, coef, hp.lr, hp.beta1, hp.beta2,
                     hp.eps, hp.weight_decay, hp.step)

    def one_core():
        g, part = step(0, n)
        _, coef = clip_coef(total([part] * P), hp.max_norm)
        update(g, 0, n, coef)

    bounds = [(k * n // cores // 8 * 8, (k + 1) * n // cores // 8 * 8 if k < cores - 1 else n)
              for k in range(cores)]
    pool = cf.ThreadPoolExecutor(max_workers=cores)

    def all_cores():
        res = list(pool.map(lambda b: step(*b), bounds))
        part = total([pt for _, pt in res])
        _, coef = clip_coef(total([part] * P), hp.max_norm)
        list(pool.map(lambda kb: update(res[kb[0]][0], kb[1][0], kb[1][1], coef),
                      enumerate(bounds)))

    def timed(fn):
        reps, t0 = 0, time.perf_counter()
        while reps < 2 or time.perf_counter() - t0 < seconds:
            fn()
            reps += 1
        return reps, time.perf_counter() - t0

    log(f"[cpu] timing the oracle step on {n} shard elements: one core, then {cores} threads")
    r1, t1 = timed(one_core)
    rk, tk = timed(all_cores)
    pool.shutdown()
    return dict(value=n * rk / tk, unit="params/s", cores=cores, kind="oracle",
                host=_cpu_model(), single_core_value=n * r1 / t1,
                sample=(f"{w.name}, owner {owner}: the first {n} elements of the shard with all "
                        f"{P} ranks' contributions; reduce-mean + norm partial + clip + AdamW "
                        f"(bf16 out) as the GPU step; {rk} repetitions in {tk:.1f} s on {cores} "
                        f"threads (one slice each) and {r1} in {t1:.1f} s on one core"))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return f"{line.split(':', 1)[1].strip()} ({os.cpu_count()} logical CPUs)"
    except OSError:
        pass
    return f"unknown ({os.cpu_count()} logical CPUs)"


# Input fills a benchmark may issue.  Every buffer is placed with one
# piece-table launch (a few per rank and per state array); a counter pass of
# rocprofv3 over a benchmark that issued ~48,000 small fill launches ended in a
# segmentation fault inside the profiler, so the many-launch fills are kept out
# of every benchmark and profiled command.
MAX_FILL_LAUNCHES = 400


def check_fill_launches(gen):
    if gen.fill_launches > MAX_FILL_LAUNCHES:
        raise RuntimeError(f"{gen.fill_launches} input fill launches (at most {MAX_FILL_LAUNCHES}): "
                           "place each buffer with one piece-table launch")


def bench_ddp(args):
    """The unsharded (DDP / NO_SHARD) step of one rank: pack its gradients,
    all-reduce mean over the P flat buffers (local arithmetic), squared norm,
    clip, AdamW over every parameter, unpack the bf16 parameters into the
    per-tensor buffers.  Prints one JSON line."""
    import numpy as np
    import torch

    import gradient_sync_zero_amd as G
    from synth import gen
    from synth import placement as PL
    from synth import workloads as W

    torch.cuda.set_device(0)
    w = W.by_id(args.config)
    P, r = w.world_size, args.owner
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    L = plan.flat_len
    need = (P + 1) * 2 * L + 2 * w.n_params + 20 * L + 2 * L
    if need > 240e9:
        print(f"bench.py: the unsharded step of {w.name} needs {need / 1e9:.0f} GB of HBM; "
              "use a smaller --config", file=sys.stderr)
        sys.exit(2)
    gbuf = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
    flats = [torch.empty(L, dtype=torch.uint16, device="cuda") for _ in range(P)]
    for q in range(P - 1, -1, -1):
        if q != r:
            _, views = PL.rank_grads(w, q, gbuf)
            G.bucket_pack(plan, views, flats[q])
    _, my_grads = PL.rank_grads(w, r, gbuf)
    master, m, v = PL.full_state(plan, w)
    check_fill_launches(gen)
    g = torch.empty(L, dtype=torch.float32, device="cuda")
    pflat = torch.empty(L, dtype=torch.uint16, device="cuda")
    pbuf = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
    params = [pbuf[s0:s0 + n] for s0, n in zip(PL.prefix(w.numel), w.numel)]
    # the all-reduce writes the P chunk owners' norm partials in the same pass
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    parts = torch.zeros(P, dtype=torch.float64, device="cuda")
    coef = torch.empty(1, dtype=torch.float32, device="cuda")
    names = ["bucket_pack", "allreduce_mean", "clip_coef", "adamw_step", "bucket_unpack"]

    def step(e=None):
        calls = [lambda: G.bucket_pack(plan, my_grads, flats[r]),
                 lambda: G.allreduce_mean(plan, flats, g, parts, ws),
                 lambda: G.clip_coef(parts, w.hp.max_norm, coef),
                 lambda: G.adamw_step(master, m, v, g, coef, w.hp, pflat),
                 lambda: G.bucket_unpack(plan, pflat, params)]
        for i, c in enumerate(calls):
            if e: e[i].record()
            c()
        if e: e[len(calls)].record()

    for _ in range(args.warmup):
        step()
    ms_step, gpu_ms, samples, step_gpu = timed_steps(step, names, args.steps)
    step_gpu = dict(timed=gpu_ms, with_call_events=step_gpu)
    per = {n: float(np.mean(v)) for n, v in samples.items()}
    byts = {"bucket_pack": 4 * w.n_params + 2 * (L - w.n_params),
            "allreduce_mean": (2 * P + 4) * L, "clip_coef": 8 * P + 12,
            "adamw_step": 30 * L, "bucket_unpack": 4 * w.n_params}
    # the all-reduce is P launches (one per chunk owner), pack and unpack one per
    # 256 tensors, the others one
    launches = {"bucket_pack": -(-len(w.numel) // 256),
                "allreduce_mean": P, "clip_coef": 1, "adamw_step": 1,
                "bucket_unpack": -(-len(w.numel) // 256)}
    kern = {n: dict(ms=per[n], ms_median=float(np.median(samples[n])), ms_min=float(np.min(samples[n])),
                    launches=launches[n], bytes=byts[n], GBps=byts[n] / (per[n] * 1e-3) / 1e9)
            for n in names}
    for n in names:
        kern[n]["frac"] = kern[n]["GBps"] / HBM_PEAK_GBPS
    # roofline: the longer of the all-reduce and the replicated AdamW
    dom = max(("allreduce_mean", "adamw_step"), key=lambda n: per[n])
    dom_bytes = byts[dom] / launches[dom]
    dom_ms = per[dom] / launches[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    kernel_symbol = {"allreduce_mean": "k_allreduce_mean", "adamw_step": "k_adamw"}[dom]
    roofline = {"bound": "hbm", "kernel": kernel_symbol, "achieved": achieved,
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                "traffic": read_traffic(kernel_symbol, profile_name(w.name, "ddp")),
                "bytes_per_launch": dom_bytes, "ms_per_launch": dom_ms}
    step_gbps = sum(byts.values()) / (ms_step * 1e-3) / 1e9
    # the plain copy (the practical ceiling and the calibration kernel of the
    # counter runs), after the timed steps as in the sharded bench
    nb = int(args.copy_gib * (1 << 30)) // 16 * 16
    a = torch.empty(nb // 4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(2):
        gen.dev_copy(a, b, nb)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        gen.dev_copy(a, b, nb)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * nb / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
    del a, b
    log(f"[gpu] DDP {w.name}: {ms_step:.3f} ms/step; " + "; ".join(
        f"{n} {kern[n]['ms']:.3f} ms {kern[n]['GBps']:.0f} GB/s" for n in names))
    print(json.dumps({
        "metric": "params/s and achieved HBM GB/s for the unsharded (DDP) step of one rank",
        "value": w.n_params / (ms_step * 1e-3), "unit": "params/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "variant": "ddp", "world_size_P": P,
                   "total_params": w.n_params, "step": " + ".join(names)},
        "hbm_GBps": step_gbps, "hbm_frac_of_peak": step_gbps / HBM_PEAK_GBPS,
        "step_ms_gpu": step_gpu, "copy_ceiling_GBps": copy_gbps, "kernels": kern,
        "roofline": roofline}),
        flush=True)


def main():
    args = parse()
    if args.summarize_counters:
        from synth import workloads as W
        if not args.command:
            sys.exit("--summarize-counters needs --command (the rocprofv3 command line)")
        summarize_counters(args.summarize_counters[0], W.by_id(args.config).name, args.command,
                           args.summarize_counters[1])
        return
    if args.summarize_trace or args.summarize_pmc:
        from synth import workloads as W
        wname = profile_name(W.by_id(args.config).name, args.variant, args.layout)
        if args.summarize_trace:
            d = _raw_dir(args.summarize_trace)
            summarize_trace(args.summarize_trace, wname,
                            args.command or profile_commands(args.config, d, d, d, args.variant,
                                                             args.layout)["trace"])
        if args.summarize_pmc:
            nb = int(args.copy_gib * (1 << 30)) // 16 * 16
            cmds = profile_commands(args.config, None, _raw_dir(args.summarize_pmc[0]),
                                    _raw_dir(args.summarize_pmc[1]), args.variant, args.layout)
            summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], wname,
                          args.command or f"{cmds['fetch']} ; {cmds['write']}", nb)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: only --gpus 1 is supported: the P data-parallel ranks are simulated "
              "as P contribution buffers on one GPU; the multi-GPU exchange is not built.",
              file=sys.stderr)
        sys.exit(2)
    ensure_built()
    if args.variant == "ddp":
        return bench_ddp(args)
    import numpy as np
    import torch

    import gradient_sync_zero_amd as G
    from synth import gen
    from synth import placement as PL
    from synth import workloads as W

    torch.cuda.set_device(0)
    w = W.by_id(args.config)
    P, r = w.world_size, args.owner
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    S, L = plan.shard_len, plan.flat_len
    dev = torch.cuda.get_device_properties(0)
    log(f"[gpu] {dev.name} ({getattr(dev, 'gcnArchName', '?')}), {w.name}: "
        f"Psi={w.n_params} S={S} flat={L} buckets={plan.n_buckets}")

    # Inputs.  The contributions are the P ranks' whole bucket-major flat
    # buffers when they fit next to the state (every workload up to the 7B
    # share), else the shard-compact buffers the P ranks send to this owner (the
    # 70B share: 64 buffers of S elements, 138 GB), or on request one
    # rank-interleaved receive buffer.  The timed step is the metric's:
    # reduce-mean (+ norm partial), clip coefficient, AdamW.
    layout = args.layout
    if layout == "auto":
        fits = (P + 2) * 2 * L + 2 * w.n_params + 18 * S < 240e9
        layout = "flat" if fits else "compact"
    t0 = time.perf_counter()
    my_grads = None
    if layout == "flat":
        gbuf = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
        flats = [torch.empty(L, dtype=torch.uint16, device="cuda") for _ in range(P)]
        for q in [q for q in range(P - 1, -1, -1) if q != r] + [r]:
            _, views = PL.rank_grads(w, q, gbuf)
            G.bucket_pack(plan, views, flats[q])
        contribs, lay = flats, G.LAYOUT_BUCKET_FLAT
        my_grads = views                          # the owner's own per-tensor gradients (filled last)
        gathered, shard_out = torch.zeros(L, dtype=torch.uint16, device="cuda"), None
    elif layout == "compact":
        contribs, lay = PL.compact_contribs(plan, w, r), G.LAYOUT_SHARD_COMPACT
        gathered, shard_out = None, torch.zeros(S, dtype=torch.uint16, device="cuda")
    else:
        contribs = [PL.interleaved_contribs(plan, w, r, G.interleaved_len(plan))]
        lay = G.LAYOUT_RANK_INTERLEAVED
        gathered, shard_out = None, torch.zeros(S, dtype=torch.uint16, device="cuda")
    master, m, v = PL.owner_state(plan, w, r)
    check_fill_launches(gen)
    g = torch.empty(S, dtype=torch.float32, device="cuda")
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    partials = torch.zeros(P, dtype=torch.float64, device="cuda")
    coef = torch.empty(1, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log(f"[gpu] inputs ready in {time.perf_counter() - t0:.1f} s ({layout} contributions, "
        f"{gen.fill_launches} fill launches); {torch.cuda.memory_allocated() / 1e9:.1f} GB allocated")

    # The other ranks' partials come from the exchange that one GPU does not
    # perform; they are stand-ins equal to this shard's partial.
    G.shard_reduce_mean(plan, r, contribs, lay, g, partials[r:r + 1], ws)
    torch.cuda.synchronize()
    partials.fill_(float(partials[r]))

    names = ["shard_reduce_mean", "clip_coef", "shard_adamw_step"]
    calls = [lambda: G.shard_reduce_mean(plan, r, contribs, lay, g, partials[r:r + 1], ws),
             lambda: G.clip_coef(partials, w.hp.max_norm, coef),
             lambda: G.shard_adamw_step(plan, r, master, m, v, g, coef, w.hp, gathered, shard_out)]
    def step(e=None):
        for k, c in enumerate(calls):
            if e: e[k].record()
            c()
        if e: e[len(calls)].record()

    for _ in range(args.warmup):
        step()
    ms_step, gpu_ms, samples, step_gpu = timed_steps(step, names, args.steps)
    step_gpu = dict(timed=gpu_ms, with_call_events=step_gpu)
    per = {n: float(np.mean(v)) for n, v in samples.items()}

    graph_ms = None
    if not args.no_graph:
        graph_ms = graph_steps(step, args.warmup, args.steps)
        log(f"[gpu] captured step: {graph_ms:.3f} ms/step over {args.steps} replays")

    # Algorithmic bytes (what the method must move), per call: the step's
    # (2P + 34) bytes per shard element.
    byts = {"shard_reduce_mean": (2 * P + 4) * S, "clip_coef": 8 * P + 12,
            "shard_adamw_step": 30 * S}
    step_bytes = sum(byts.values())
    kern = {n: dict(ms=per[n], ms_median=float(np.median(samples[n])),
                    ms_min=float(np.min(samples[n])), launches=1,
                    GBps=byts[n] / (per[n] * 1e-3) / 1e9, bytes=byts[n]) for n in names}
    for n in names:
        kern[n]["frac"] = kern[n]["GBps"] / HBM_PEAK_GBPS
    # The roofline names the longer of the step's two data kernels.
    dom = max(("shard_reduce_mean", "shard_adamw_step"), key=lambda n: per[n])
    dom_bytes, dom_ms = byts[dom], per[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    kernel_symbol = {"shard_reduce_mean": reduce_kernel(P, S, layout),
                     "shard_adamw_step": "k_adamw"}[dom]
    traffic = read_traffic(kernel_symbol, profile_name(w.name, "zero", layout))
    step_gbps = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"[gpu] {ms_step:.3f} ms/step, {step_gbps:.0f} GB/s; " + "; ".join(
        f"{n} {kern[n]['ms']:.3f} ms {kern[n]['GBps']:.0f} GB/s" for n in names))

    def time_call(fn, reps=5):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # The other rows of the path, standalone: the pack (the first part of the
    # rank's share; in the flat layout the owner's own gradients into its flat
    # buffer, otherwise a window of the model that fits beside the 138 GB of
    # contributions), the squared norm of g (fused into the reduce on the
    # step), the all-gather layout writer (fused into the AdamW store), and the
    # rows beyond the step.
    shard_bf16 = torch.zeros(S, dtype=torch.uint16, device="cuda")
    part1 = torch.zeros(1, dtype=torch.float64, device="cuda")
    g_step = g.clone()                 # the step's reduced gradient, kept for the layout check
    standalone = {}
    rows = [("shard_grad_sqnorm", lambda: G.shard_grad_sqnorm(g, part1, ws), 4 * S),
            ("shard_reduce_mean_bf16_wire",
             lambda: G.shard_reduce_mean(plan, r, contribs, lay, g, part1, ws, bf16_wire=True),
             (2 * P + 4) * S)]
    if my_grads is not None:
        rows.append(("bucket_pack", lambda: G.bucket_pack(plan, my_grads, contribs[r]),
                     4 * w.n_params + 2 * (L - w.n_params)))
        rows.append(("allgather_layout_write",
                     lambda: G.allgather_layout_write(plan, r, shard_bf16, gathered), 4 * S))
        rows.append(("bucket_accumulate",
                     lambda: G.bucket_accumulate(plan, my_grads, contribs[r]), 6 * w.n_params))
    else:
        # The owner's pack on a window of the model: the trailing tensors that
        # fill its first 20 buckets (the plan of those tensors alone has the same
        # buckets).
        nb_win = min(20, plan.n_buckets)
        last = plan.bucket(nb_win - 1)
        t_min = last["first_tensor"] - last["n_tensors"] + 1
        wplan = G.Plan(w.numel[t_min:], w.bucket_cap_bytes, P).upload()
        wn = sum(w.numel[t_min:])
        wbuf = torch.empty(wn, dtype=torch.uint16, device="cuda")
        wgrads = list(torch.split(wbuf, w.numel[t_min:]))
        PL.fill_pieces(wbuf, [(0, sum(w.numel[:t_min]), wn)], w, W.KIND_GRAD, r, w.grad_std,
                       gen.MODE_BF16)
        wflat = torch.empty(wplan.flat_len, dtype=torch.uint16, device="cuda")
        rows.append((f"bucket_pack_window{nb_win}",
                     lambda: G.bucket_pack(wplan, wgrads, wflat),
                     4 * wn + 2 * (wplan.flat_len - wn)))
        log(f"[gpu] pack window: the first {nb_win} buckets, tensors {t_min}..{len(w.numel) - 1}, "
            f"{wn} params")
    check_fill_launches(gen)
    for name, fn, nbytes in rows:
        ms = time_call(fn)
        standalone[name] = dict(ms=ms, bytes=nbytes, GBps=nbytes / (ms * 1e-3) / 1e9,
                                frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS)
    # fp32 accumulation buckets and the reduce over fp32 contributions, when
    # their buffers fit beside the working set.
    if my_grads is not None and 4 * L < 0.8 * torch.cuda.mem_get_info()[0]:
        f32 = torch.zeros(L, dtype=torch.float32, device="cuda")
        G.bucket_pack_f32(plan, my_grads, f32)
        ms = time_call(lambda: G.bucket_accumulate_f32(plan, my_grads, f32))
        nbytes = 10 * w.n_params
        standalone["bucket_accumulate_f32"] = dict(ms=ms, bytes=nbytes,
                                                   GBps=nbytes / (ms * 1e-3) / 1e9,
                                                   frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS)
        del f32
    if 4 * P * S < 0.8 * torch.cuda.mem_get_info()[0]:
        c32 = [g.clone() for _ in range(P)]      # values do not change the timing
        ms = time_call(lambda: G.shard_reduce_mean_f32(plan, r, c32, G.LAYOUT_SHARD_COMPACT, g,
                                                       part1, ws))
        nbytes = (4 * P + 4) * S
        standalone["shard_reduce_mean_f32"] = dict(ms=ms, bytes=nbytes,
                                                   GBps=nbytes / (ms * 1e-3) / 1e9,
                                                   frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS)
        del c32
    log("[gpu] standalone: " + "; ".join(f"{n} {v['ms']:.3f} ms {v['GBps']:.0f} GB/s"
                                         for n, v in standalone.items()))
    del shard_bf16

    # The reduce's own read pattern without arithmetic: the first 2*S bytes of
    # each of the P contribution buffers read at the same offsets (or the one
    # interleaved buffer read straight through).
    nbs = 2 * S // 16 * 16
    sink = torch.empty(max(gen.probe_out_words(nbs), gen.probe_out_words(P * nbs)),
                       dtype=torch.int32, device="cuda")
    ceil = {}

    def probe(name, fn, nbytes):
        for _ in range(2):
            fn()
        ceil[name] = nbytes / (time_call(fn, reps=10) * 1e-3) / 1e9

    if layout == "interleaved":
        probe("read_interleaved", lambda: gen.dev_read(contribs[0], sink, P * nbs), P * nbs)
    else:
        probe(f"read_{P}_streams", lambda: gen.dev_read_streams(contribs, nbs, sink), P * nbs)

    # The other receive layout, timed in the same process when both do not fit
    # at once: the reduce (with its norm partial) over the same values in one
    # rank-interleaved buffer, its result checked bit for bit against the
    # step's g.  Allocated after the first layout's buffers are freed.
    other = None
    if layout in ("compact", "flat") and not args.no_interleaved:
        del contribs
        if layout == "flat":
            del flats, gbuf, views, my_grads
        torch.cuda.empty_cache()
        ibuf = PL.interleaved_contribs(plan, w, r, G.interleaved_len(plan))
        check_fill_launches(gen)
        icall = lambda: G.shard_reduce_mean(plan, r, [ibuf], G.LAYOUT_RANK_INTERLEAVED, g,  # noqa: E731
                                            part1, ws)
        icall()
        torch.cuda.synchronize()
        same = bool(torch.equal(g.view(torch.int32), g_step.view(torch.int32)))
        ims = time_call(icall, reps=max(5, args.steps // 2))
        probe("read_interleaved", lambda: gen.dev_read(ibuf, sink, P * nbs), P * nbs)
        nbytes = (2 * P + 4) * S
        fused = ims + per["clip_coef"] + per["shard_adamw_step"]
        other = {"layout": "rank-interleaved (one receive buffer, 512-element pieces per rank)",
                 "shard_reduce_mean": dict(ms=ims, bytes=nbytes, GBps=nbytes / (ims * 1e-3) / 1e9,
                                           frac=nbytes / (ims * 1e-3) / 1e9 / HBM_PEAK_GBPS),
                 "g_bit_identical_to_step": same,
                 "step_ms_with_this_reduce": fused,
                 "step_frac_with_this_reduce": step_bytes / (fused * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        log(f"[gpu] interleaved receive buffer: reduce {ims:.3f} ms "
            f"{nbytes / (ims * 1e-3) / 1e9:.0f} GB/s, g identical: {same}")
        del ibuf
        torch.cuda.empty_cache()
    else:
        del contribs
    del sink, g_step

    # Plain streaming probes in the kernels' launch shape, run after the timed
    # steps so that their allocations do not fragment the memory the working set
    # was placed in: copy (the practical ceiling for half-read/half-write traffic
    # and the calibration kernel of the counter runs), read-only and write-only.
    nb = int(args.copy_gib * (1 << 30)) // 16 * 16
    a = torch.empty(nb // 4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    sink = torch.empty(gen.probe_out_words(nb), dtype=torch.int32, device="cuda")
    probe("copy", lambda: gen.dev_copy(a, b, nb), 2 * nb)
    probe("read", lambda: gen.dev_read(a, sink, nb), nb)
    probe("write", lambda: gen.dev_write(b, nb), nb)
    del a, b, sink
    log("[gpu] streaming ceilings (GB/s): " + ", ".join(f"{k} {v:.0f}" for k, v in ceil.items()))

    cpu = None if args.no_cpu_baseline else cpu_baseline(w, r)
    out = {
        "metric": METRIC,
        "value": S / (ms_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "world_size_P": P, "owner": r, "total_params": w.n_params,
                   "shard_params": S, "bucket_cap_MiB": w.bucket_cap_bytes // (1 << 20),
                   "buckets": plan.n_buckets,
                   "contribution_layout": {"flat": "bucket-flat", "compact": "shard-compact",
                                           "interleaved": "rank-interleaved"}[layout],
                   "precision": "bf16 grads/params, fp32 accumulation and master/m/v",
                   "step": " + ".join(names) + (" (all-gather layout)" if gathered is not None
                                                 else " (shard-layout bf16)")},
        "graph_ms_per_step": graph_ms,
        "graph_hbm_frac_of_peak": (None if graph_ms is None else
                                   step_bytes / (graph_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS),
        "step_ms_gpu": step_gpu,
        "hbm_GBps": step_gbps,
        "hbm_frac_of_peak": step_gbps / HBM_PEAK_GBPS,
        "step_bytes": step_bytes,
        "copy_ceiling_GBps": ceil["copy"],
        "streaming_ceilings_GBps": ceil,
        "kernels": kern,
        "kernels_standalone": standalone,
        "other_layout": other,
        "roofline": {"bound": "hbm", "kernel": kernel_symbol, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "bytes_per_launch": dom_bytes,
                     "ms_per_launch": dom_ms},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
