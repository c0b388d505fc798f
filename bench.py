#!/usr/bin/env python3
"""Benchmark of one rank's share of a synchronous data-parallel step on one
MI355X: bucket pack -> ring-order reduce-mean (+ squared-norm partial) ->
clip coefficient -> AdamW writing bf16 parameters in all-gather layout.

Workload (default): the 7B Llama-shaped share -- 6,738,415,616 parameters in
291 tensors, P = 8 simulated ranks, 25 MiB buckets, owner 0's shard of
842,301,952 elements.  All P ranks' bucket-major gradient buffers are resident
in HBM; each timed step packs owner 0's per-tensor gradients into its own flat
buffer, reduces owner 0's chunks over the 8 flat buffers, forms the clip
coefficient, and updates the shard's fp32 master/m/v in place.

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
    ap.add_argument("--config", type=int, default=3, help="workload id (synth.workloads)")
    ap.add_argument("--owner", type=int, default=0)
    ap.add_argument("--variant", choices=["zero", "ddp"], default="zero",
                    help="zero: the ZeRO-1/2 shard step (default); ddp: the unsharded step "
                         "(all-reduce, replicated AdamW, unpack)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured as one HIP graph (graph_ms_per_step)")
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


def short_name(full):
    # template instances that move different bytes get their own names
    if "k_pack<1>" in full:
        return "k_unpack"
    if "k_pack<2>" in full:
        return "k_accumulate"
    if "k_reduce_mean<" in full:
        args = [a.strip() for a in full.split("k_reduce_mean<")[1].split(">")[0].split(",")]
        if len(args) == 5 and args[4] == "true":
            return "k_reduce_mean_bf16_wire"
        if len(args) >= 4 and args[3] == "true":
            return "k_allreduce_mean"
    if "k_reduce_mean_lc<" in full:          # <T, PS, NORM, FLAT, OUTFLAT, W16>
        args = [a.strip() for a in full.split("k_reduce_mean_lc<")[1].split(">")[0].split(",")]
        if args[0] == "float":
            return "k_reduce_mean_f32"
        if len(args) == 6 and args[5] == "true":
            return "k_reduce_mean_bf16_wire"
        if len(args) == 6 and args[4] == "true":
            return "k_allreduce_mean"
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


def profile_commands(config, trace_dir, fetch_dir, write_dir, variant="zero"):
    """The rocprofv3 command lines (run from the repository root) whose output
    the summaries below are made from: a kernel trace of the default bench of
    a workload, and one counter pass each for FETCH_SIZE and WRITE_SIZE, each
    writing <dir>/bench_*.csv."""
    var = " --variant ddp" if variant == "ddp" else ""
    bench_args = f"python3 bench.py --config {config}{var} --no-cpu-baseline"
    short = f"python3 bench.py --config {config}{var} --steps 3 --warmup 1 --no-cpu-baseline"
    return {"trace": f"rocprofv3 --kernel-trace --stats -f csv -d {trace_dir} "
                     f"-o bench -- {bench_args}",
            "fetch": f"rocprofv3 --pmc FETCH_SIZE -f csv -d {fetch_dir} -o bench -- {short}",
            "write": f"rocprofv3 --pmc WRITE_SIZE -f csv -d {write_dir} -o bench -- {short}"}


def profile_name(workload, variant):
    """Name of a workload's profile summaries: the unsharded (DDP) step gets
    its own files."""
    return f"{workload}-ddp" if variant == "ddp" else workload


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


def kernel_source_digest():
    """SHA-256 over the library's kernel sources (names and contents), the key
    that ties a counter summary to the kernels it measured."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(name.encode() + b"\0")
        h.update(open(os.path.join(ROOT, "gradient_sync_zero_amd", "csrc", name), "rb").read())
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


def cpu_baseline(w, owner):
    """The oracle as it stands, on one core, over the trailing buckets of the
    same workload (the first buckets of its plan): owner's pack, reduce-mean,
    squared norm, clip and AdamW + all-gather layout.  Input generation is not
    timed."""
    import numpy as np
    from oracle import pack as opack
    from oracle.adamw import adamw
    from oracle.layout import ag_write
    from oracle.norm import clip_coef, sqnorm_partial, total
    from oracle.plan import make_plan
    from oracle.reduce import reduce_mean
    from synth import gen
    from synth import workloads as W

    numel = w.numel
    m, s = 0, 0
    while s < 256_000_000 and m < len(numel):
        m += 1
        s += numel[-m]
    sub = numel[-m:]
    pre = sum(numel[:-m])
    P = w.world_size
    plan = make_plan(sub, w.bucket_cap_bytes, P)
    offs = np.cumsum([0] + sub)
    log(f"[cpu] generating the oracle sample: {len(plan.buckets)} buckets, {s} params x {P} ranks")
    grads = []
    for q in range(P):
        G = gen.host_fill(w.cfg_id, W.KIND_GRAD, q, pre, s, w.grad_std, gen.MODE_BF16)
        grads.append([G[offs[i]:offs[i + 1]] for i in range(m)])
    others = [opack.pack(plan, grads[q]) for q in range(P) if q != owner]
    S = plan.shard_len
    state = []
    for kind, std, mode in ((W.KIND_MASTER, W.MASTER_STD, gen.MODE_F32),
                            (W.KIND_EXP_AVG, W.EXP_AVG_STD, gen.MODE_F32),
                            (W.KIND_EXP_AVG_SQ, W.EXP_AVG_SQ_STD, gen.MODE_ABS)):
        state.append(gen.host_fill(w.cfg_id, kind, 0, pre, S, std, mode))
    hp = w.hp
    log(f"[cpu] timing the oracle step on S = {S} shard elements")

    def one_step():
        mine = opack.pack(plan, grads[owner])
        flats = others[:owner] + [mine] + others[owner:]
        g = reduce_mean([opack.owner_view(plan, f, owner) for f in flats], owner)
        part = sqnorm_partial(g)
        _, coef = clip_coef(total([part] * P), hp.max_norm)
        th, m1, v1, p = adamw(state[0], state[1], state[2], g, coef, hp.lr, hp.beta1, hp.beta2,
                              hp.eps, hp.weight_decay, hp.step)
        gathered = np.zeros(plan.flat_len, dtype=np.uint16)
        ag_write(plan, owner, p, gathered)

    # the same step on the same inputs, repeated until about 10 s of CPU work
    reps, t0 = 0, time.perf_counter()
    while reps < 3 or time.perf_counter() - t0 < 10.0:
        one_step()
        reps += 1
    dt = time.perf_counter() - t0
    return dict(value=S * reps / dt, unit="params/s", cores=1, kind="oracle",
                host=_cpu_model(),
                sample=(f"{w.name}: the first {len(plan.buckets)} buckets of the plan "
                        f"({m} trailing tensors, {s} params, owner {owner} shard of {S}); "
                        f"pack + reduce-mean + norm + clip + AdamW + all-gather layout, "
                        f"{reps} repetitions in {dt:.1f} s of single-threaded NumPy"))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return f"{line.split(':', 1)[1].strip()} ({os.cpu_count()} logical CPUs)"
    except OSError:
        pass
    return f"unknown ({os.cpu_count()} logical CPUs)"


def bench_ddp(args):
    """The unsharded (DDP / NO_SHARD) step of one rank: pack its gradients,
    all-reduce mean over the P flat buffers (local arithmetic), squared norm,
    clip, AdamW over every parameter, unpack the bf16 parameters into the
    per-tensor buffers.  Prints one JSON line."""
    import numpy as np
    import torch

    import gradient_sync_zero_amd as G
    from synth import workloads as W
    from tests import gpu_inputs as GI

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
            _, views = GI.rank_grads(w, q, gbuf)
            G.bucket_pack(plan, views, flats[q])
    _, my_grads = GI.rank_grads(w, r, gbuf)
    master, m, v = GI.full_state(plan, w)
    g = torch.empty(L, dtype=torch.float32, device="cuda")
    pflat = torch.empty(L, dtype=torch.uint16, device="cuda")
    pbuf = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
    params = [pbuf[s0:s0 + n] for s0, n in zip(GI.prefix(w.numel), w.numel)]
    # the all-reduce writes the P chunk owners' norm partials in the same pass
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    parts = torch.zeros(P, dtype=torch.float64, device="cuda")
    coef = torch.empty(1, dtype=torch.float32, device="cuda")
    names = ["bucket_pack", "allreduce_mean", "clip_coef", "adamw_step", "bucket_unpack"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
          for _ in range(args.steps)]

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
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / args.steps * 1e3
    samples = {n: [ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(args.steps)]
               for i, n in enumerate(names)}
    per = {n: float(np.mean(v)) for n, v in samples.items()}
    step_gpu = gpu_step_stats(ev)
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
    from synth import gen
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
                   "model_params": w.n_params, "step": " + ".join(names)},
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
        wname = profile_name(W.by_id(args.config).name, args.variant)
        if args.summarize_trace:
            d = _raw_dir(args.summarize_trace)
            summarize_trace(args.summarize_trace, wname,
                            args.command or profile_commands(args.config, d, d, d,
                                                             args.variant)["trace"])
        if args.summarize_pmc:
            nb = int(args.copy_gib * (1 << 30)) // 16 * 16
            cmds = profile_commands(args.config, None, _raw_dir(args.summarize_pmc[0]),
                                    _raw_dir(args.summarize_pmc[1]), args.variant)
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
    from synth import workloads as W
    from tests import gpu_inputs as GI

    torch.cuda.set_device(0)
    w = W.by_id(args.config)
    P, r = w.world_size, args.owner
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    S, L = plan.shard_len, plan.flat_len
    dev = torch.cuda.get_device_properties(0)
    log(f"[gpu] {dev.name} ({getattr(dev, 'gcnArchName', '?')}), {w.name}: "
        f"Psi={w.n_params} S={S} flat={L} buckets={plan.n_buckets}")

    # Inputs.  When all P ranks' bucket-major flat buffers fit next to the
    # state (every config but the 70B share), the step packs the owner's own
    # per-tensor gradients and reduces over the P flat buffers.  Otherwise the
    # contributions are the shard-compact buffers the P ranks send to this
    # owner, and the step is the reduce + clip + AdamW the metric names (the
    # owner's full-model pack would need 2 x 138 GB more than the GPU holds).
    t0 = time.perf_counter()
    flat_mode = (P + 2) * 2 * L + 2 * w.n_params + 18 * S < 240e9
    if flat_mode:
        gbuf = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
        flats = [torch.empty(L, dtype=torch.uint16, device="cuda") for _ in range(P)]
        for q in list(range(P - 1, -1, -1)):
            if q == r:
                continue
            _, views = GI.rank_grads(w, q, gbuf)
            G.bucket_pack(plan, views, flats[q])
        _, my_grads = GI.rank_grads(w, r, gbuf)      # the owner's own per-tensor gradients
        contribs, layout = flats, G.LAYOUT_BUCKET_FLAT
        gathered, shard_out = torch.zeros(L, dtype=torch.uint16, device="cuda"), None
    else:
        contribs, layout = GI.compact_contribs(plan, w, r), G.LAYOUT_SHARD_COMPACT
        gathered, shard_out = None, torch.zeros(S, dtype=torch.uint16, device="cuda")
    master, m, v = GI.owner_state(plan, w, r)
    g = torch.empty(S, dtype=torch.float32, device="cuda")
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    partials = torch.zeros(P, dtype=torch.float64, device="cuda")
    coef = torch.empty(1, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log(f"[gpu] inputs ready in {time.perf_counter() - t0:.1f} s "
        f"({'bucket-flat' if flat_mode else 'shard-compact'} contributions); "
        f"{torch.cuda.memory_allocated() / 1e9:.1f} GB allocated")

    # The other ranks' partials come from the exchange that one GPU does not
    # perform; they are stand-ins equal to this shard's partial.
    if flat_mode:
        G.bucket_pack(plan, my_grads, flats[r])
    G.shard_reduce_mean(plan, r, contribs, layout, g, partials[r:r + 1], ws)
    torch.cuda.synchronize()
    partials.fill_(float(partials[r]))

    names = (["bucket_pack"] if flat_mode else []) + ["shard_reduce_mean", "clip_coef",
                                                       "shard_adamw_step"]
    launches = {"bucket_pack": -(-plan.n_tensors // 256), "shard_reduce_mean": 1,
                "clip_coef": 1, "shard_adamw_step": 1}
    nev = len(names) + 1
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]

    def step(e=None):
        k = 0
        if e: e[k].record()
        if flat_mode:
            G.bucket_pack(plan, my_grads, flats[r])
            k += 1
            if e: e[k].record()
        G.shard_reduce_mean(plan, r, contribs, layout, g, partials[r:r + 1], ws)
        k += 1
        if e: e[k].record()
        G.clip_coef(partials, w.hp.max_norm, coef)
        k += 1
        if e: e[k].record()
        G.shard_adamw_step(plan, r, master, m, v, g, coef, w.hp, gathered, shard_out)
        k += 1
        if e: e[k].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    samples = {n: [ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(args.steps)]
               for i, n in enumerate(names)}
    per = {n: float(np.mean(v)) for n, v in samples.items()}
    step_gpu = gpu_step_stats(ev)

    graph_ms = None
    if args.graph:
        # The same step captured once into a HIP graph and replayed: the launch
        # gaps between the calls disappear (this matters for small workloads).
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) / args.steps * 1e3
        log(f"[gpu] captured step: {graph_ms:.3f} ms/step over {args.steps} replays")

    # Algorithmic bytes (what the method must move), per call.
    byts = {"bucket_pack": 4 * w.n_params + 2 * (L - w.n_params),
            "shard_reduce_mean": (2 * P + 4) * S,
            "clip_coef": 8 * P + 12,
            "shard_adamw_step": 30 * S}
    byts = {n: byts[n] for n in names}
    step_bytes = sum(byts.values())
    kern = {n: dict(ms=per[n], ms_median=float(np.median(samples[n])),
                    ms_min=float(np.min(samples[n])), launches=launches[n],
                    GBps=byts[n] / (per[n] * 1e-3) / 1e9, bytes=byts[n]) for n in names}
    for n in names:
        kern[n]["frac"] = kern[n]["GBps"] / HBM_PEAK_GBPS
    # The roofline names the longer of the metric's two kernels (reduce-mean and
    # AdamW): a stable choice, where the longest call of the step (the pack's
    # two launches and AdamW are within a few percent on the 7B share) is not.
    dom = max(("shard_reduce_mean", "shard_adamw_step"), key=lambda n: per[n])
    dom_bytes = byts[dom] / launches[dom]
    dom_ms = per[dom] / launches[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    kernel_symbol = {"bucket_pack": "k_pack", "shard_reduce_mean": "k_reduce_mean",
                     "clip_coef": "k_clip", "shard_adamw_step": "k_adamw"}[dom]
    traffic = read_traffic(kernel_symbol, w.name)
    step_gbps = step_bytes / (ms_step * 1e-3) / 1e9
    # The reduce-mean + AdamW shard step alone ((2P + 34) bytes per shard element).
    fused_ms = per["shard_reduce_mean"] + per["clip_coef"] + per["shard_adamw_step"]
    fused_gbps = (2 * P + 34) * S / (fused_ms * 1e-3) / 1e9
    log(f"[gpu] {ms_step:.3f} ms/step; " + "; ".join(
        f"{n} {kern[n]['ms']:.3f} ms {kern[n]['GBps']:.0f} GB/s" for n in names))

    # The standalone forms of two rows the step runs fused: the squared norm of
    # g (fused into the reduce) and the all-gather layout writer (fused into
    # the AdamW store).
    def time_call(fn, reps=5):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    shard_bf16 = torch.zeros(S, dtype=torch.uint16, device="cuda")
    part1 = torch.zeros(1, dtype=torch.float64, device="cuda")
    standalone = {}
    rows = [("shard_grad_sqnorm", lambda: G.shard_grad_sqnorm(g, part1, ws), 4 * S),
            ("shard_reduce_mean_bf16_wire",
             lambda: G.shard_reduce_mean(plan, r, contribs, layout, g, part1, ws, bf16_wire=True),
             (2 * P + 4) * S)]
    if gathered is not None:
        rows.append(("allgather_layout_write",
                     lambda: G.allgather_layout_write(plan, r, shard_bf16, gathered), 4 * S))
    if flat_mode:
        rows.append(("bucket_accumulate",
                     lambda: G.bucket_accumulate(plan, my_grads, flats[r]), 6 * w.n_params))
    if not flat_mode:
        # The owner's pack on a window of the model: the trailing tensors that
        # fill its first 20 buckets (the plan of those tensors alone has the same
        # buckets).  The whole model's gradients and flat buffer would not fit
        # beside the P contributions.
        nb_win = min(20, plan.n_buckets)
        last = plan.bucket(nb_win - 1)
        t_min = last["first_tensor"] - last["n_tensors"] + 1
        wplan = G.Plan(w.numel[t_min:], w.bucket_cap_bytes, P).upload()
        wn = sum(w.numel[t_min:])
        wbuf = torch.empty(wn, dtype=torch.uint16, device="cuda")
        wgrads = list(torch.split(wbuf, w.numel[t_min:]))
        GI.fill_pieces(wbuf, [(0, sum(w.numel[:t_min]), wn)], w, W.KIND_GRAD, r, w.grad_std,
                       gen.MODE_BF16)
        wflat = torch.empty(wplan.flat_len, dtype=torch.uint16, device="cuda")
        rows.append((f"bucket_pack_window{nb_win}",
                     lambda: G.bucket_pack(wplan, wgrads, wflat),
                     4 * wn + 2 * (wplan.flat_len - wn)))
        log(f"[gpu] pack window: the first {nb_win} buckets, tensors {t_min}..{len(w.numel) - 1}, "
            f"{wn} params")
    for name, fn, nbytes in rows:
        ms = time_call(fn)
        standalone[name] = dict(ms=ms, bytes=nbytes, GBps=nbytes / (ms * 1e-3) / 1e9,
                                frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS)
    # fp32 accumulation buckets and the reduce over fp32 contributions, when
    # their buffers fit beside the working set: one fp32 flat buffer for the
    # accumulation (10 bytes per parameter: bf16 gradient in, fp32 bucket in and
    # out) and P shard-compact fp32 contributions for the reduce (4P + 4 bytes
    # per shard element).
    if flat_mode and 4 * L < 0.8 * torch.cuda.mem_get_info()[0]:
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

    # Plain streaming probes in the kernels' launch shape, run after the timed
    # steps so that their allocations do not fragment the memory the working set
    # was placed in: copy (the practical ceiling for half-read/half-write traffic
    # and the calibration kernel of the counter runs), read-only and write-only.
    nb = int(args.copy_gib * (1 << 30)) // 16 * 16
    a = torch.empty(nb // 4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    # the reduce's own pattern without arithmetic: the first 2*S bytes of each
    # of the P contribution buffers, read at the same offsets
    nbs = 2 * S // 16 * 16
    sink = torch.empty(max(gen.probe_out_words(nb), gen.probe_out_words(nbs)), dtype=torch.int32,
                       device="cuda")
    ceil = {}
    for name, fn, nbytes in (("copy", lambda: gen.dev_copy(a, b, nb), 2 * nb),
                             ("read", lambda: gen.dev_read(a, sink, nb), nb),
                             ("write", lambda: gen.dev_write(b, nb), nb),
                             (f"read_{P}_streams",
                              lambda: gen.dev_read_streams(contribs, nbs, sink), P * nbs)):
        for _ in range(2):
            fn()
        ms = time_call(fn, reps=10)
        ceil[name] = nbytes / (ms * 1e-3) / 1e9
    copy_gbps = ceil["copy"]
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
        "config": {"workload": w.name, "world_size_P": P, "owner": r, "model_params": w.n_params,
                   "shard_params": S, "bucket_cap_MiB": w.bucket_cap_bytes // (1 << 20),
                   "buckets": plan.n_buckets,
                   "contribution_layout": "bucket-flat" if flat_mode else "shard-compact",
                   "precision": "bf16 grads/params, fp32 accumulation and master/m/v",
                   "step": " + ".join(names) + (" (all-gather layout)" if flat_mode
                                                 else " (shard-layout bf16)")},
        "graph_ms_per_step": graph_ms,
        "step_ms_gpu": step_gpu,
        "reduce_adamw_ms": fused_ms,
        "reduce_adamw_GBps": fused_gbps,
        "reduce_adamw_frac_of_peak": fused_gbps / HBM_PEAK_GBPS,
        "hbm_GBps": step_gbps,
        "hbm_frac_of_peak": step_gbps / HBM_PEAK_GBPS,
        "step_bytes": step_bytes,
        "copy_ceiling_GBps": copy_gbps,
        "streaming_ceilings_GBps": ceil,
        "kernels_standalone": standalone,
        "kernels": kern,
        "roofline": {"bound": "hbm", "kernel": kernel_symbol, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "bytes_per_launch": dom_bytes,
                     "ms_per_launch": dom_ms},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
