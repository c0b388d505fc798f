"""GPU parity of two rows beyond the shard step: gradient accumulation into the
bucket buffer over micro-batches, and the reduce with bf16 partial sums on the
wire -- bit for bit against the oracle -- plus the drift of the bf16 wire from
the fp32-accumulated mean (reported, and bounded as the oracle's pin bounds it)."""
import numpy as np
import pytest
import torch

import gradient_sync_zero_amd as G
from oracle import pack as opack
from oracle.bf16 import widen
from oracle.norm import sqnorm_partial
from oracle.plan import make_plan
from oracle.reduce import reduce_mean, reduce_mean_bf16_wire
from synth import gen
from synth import workloads as W
from tests import gpu_inputs as GI
from tests import oracle_inputs as OI
from tests.parity import bf16_wire_bound, assert_bits, host

pytestmark = pytest.mark.gpu

MICRO = 1000    # generator rank field of micro-batch k of rank 0: MICRO + k


def micro_grads_dev(w, k):
    pre = GI.prefix(w.numel)
    out = []
    for s0, n in zip(pre, w.numel):
        t = torch.empty(n, dtype=torch.uint16, device="cuda")
        if n:
            gen.dev_fill(t, w.cfg_id, W.KIND_GRAD, MICRO + k, s0, w.grad_std, gen.MODE_BF16)
        out.append(t)
    return out


def micro_grads_host(w, k):
    flat = gen.host_fill(w.cfg_id, W.KIND_GRAD, MICRO + k, 0, w.n_params, w.grad_std,
                         gen.MODE_BF16)
    pre = GI.prefix(w.numel)
    return [flat[s0:s0 + n] for s0, n in zip(pre, w.numel)]


@pytest.mark.parametrize("cfg", [0, 1])
def test_gradient_accumulation_over_micro_batches(cfg):
    w = W.by_id(cfg)
    plan = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, w.world_size)
    flat = torch.full((plan.flat_len,), 0x7777, dtype=torch.uint16, device="cuda")
    G.bucket_pack(plan, micro_grads_dev(w, 0), flat)
    for k in (1, 2, 3):
        G.bucket_accumulate(plan, micro_grads_dev(w, k), flat)
    torch.cuda.synchronize()
    ref = opack.pack(oplan, micro_grads_host(w, 0))
    for k in (1, 2, 3):
        ref = opack.accumulate(oplan, ref, micro_grads_host(w, k))
    assert_bits(host(flat), ref, f"{w.name}: bucket after 4 micro-batches")


@pytest.mark.parametrize("cfg", [0, 1])
def test_bf16_wire_reduce_all_owners(cfg):
    w = W.by_id(cfg)
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    flats = []
    for q in range(P):
        f = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, GI.rank_grads_separate(w, q), f)
        flats.append(f)
    oflats = [OI.rank_flat(oplan, w, q) for q in range(P)]
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    part = torch.zeros(1, dtype=torch.float64, device="cuda")
    worst, changed, n_all = 0.0, 0, 0
    for r in range(P):
        g = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
        G.shard_reduce_mean(plan, r, flats, G.LAYOUT_BUCKET_FLAT, g, part, ws, bf16_wire=True)
        gc = torch.empty_like(g)
        comp = GI.compact_contribs(plan, w, r)
        G.shard_reduce_mean(plan, r, comp, G.LAYOUT_SHARD_COMPACT, gc, None, None, bf16_wire=True)
        torch.cuda.synchronize()
        cs = [opack.owner_view(oplan, f, r) for f in oflats]
        ref = reduce_mean_bf16_wire(cs, r)
        assert_bits(host(g), ref, f"bf16-wire g owner {r}")
        assert_bits(host(gc), ref, f"bf16-wire g owner {r} (shard-compact)")
        assert abs(host(part)[0] - sqnorm_partial(ref)) <= 1e-12 * sqnorm_partial(ref)
        fp32 = reduce_mean(cs, r).astype(np.float64)
        abs_sum = np.sum([np.abs(widen(c)).astype(np.float64) for c in cs], axis=0)
        bound = bf16_wire_bound(abs_sum, P)
        err = np.abs(fp32 - ref)
        assert (err <= bound * (1 + 1e-12)).all()
        worst = max(worst, float((err / np.maximum(bound, 1e-300)).max()))
        changed += int((err > 0).sum())
        n_all += err.size
    print(f"[{w.name}] bf16 wire vs fp32 accumulation: {changed / n_all:.1%} of elements differ; "
          f"largest difference {worst:.2f} of the rounding bound", flush=True)


# --- fp32 accumulation buckets and the fp32-contribution reduce -------------

MICRO_F32 = 1100    # generator rank field of rank q's micro-batch k: MICRO_F32 + 8q + k


def rank_micro_dev(w, q, k):
    out = []
    for s0, n in zip(GI.prefix(w.numel), w.numel):
        t = torch.empty(n, dtype=torch.uint16, device="cuda")
        if n:
            gen.dev_fill(t, w.cfg_id, W.KIND_GRAD, MICRO_F32 + 8 * q + k, s0, w.grad_std,
                         gen.MODE_BF16)
        out.append(t)
    return out


def rank_micro_host(w, q, k):
    flat = gen.host_fill(w.cfg_id, W.KIND_GRAD, MICRO_F32 + 8 * q + k, 0, w.n_params,
                         w.grad_std, gen.MODE_BF16)
    return [flat[s0:s0 + n] for s0, n in zip(OI.prefix(w.numel), w.numel)]


def compact_from_flat(plan, flat, r):
    """Owner r's chunks of a device flat buffer, in shard order (library plan)."""
    return torch.cat([flat[b["base"] + r * b["chunk"]:b["base"] + (r + 1) * b["chunk"]]
                      for b in plan.buckets()]).contiguous()


@pytest.mark.parametrize("cfg,micro,owners", [(0, 4, None), (1, 2, (0, 7))])
def test_fp32_accumulation_then_fp32_reduce(cfg, micro, owners):
    w = W.by_id(cfg)
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    dev, ref = [], []
    for q in range(P):
        f = torch.full((plan.flat_len,), float("nan"), dtype=torch.float32, device="cuda")
        G.bucket_pack_f32(plan, rank_micro_dev(w, q, 0), f)      # also writes the pads
        for k in range(1, micro):
            G.bucket_accumulate_f32(plan, rank_micro_dev(w, q, k), f)
        o = opack.pack_f32(oplan, rank_micro_host(w, q, 0))
        for k in range(1, micro):
            o = opack.accumulate_f32(oplan, o, rank_micro_host(w, q, k))
        dev.append(f)
        ref.append(o)
    torch.cuda.synchronize()
    for q in range(P):
        assert_bits(host(dev[q]), ref[q], f"{w.name}: fp32 buckets of rank {q}")
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    part = torch.zeros(1, dtype=torch.float64, device="cuda")
    for r in (owners or range(P)):
        g = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
        G.shard_reduce_mean_f32(plan, r, dev, G.LAYOUT_BUCKET_FLAT, g, part, ws)
        gc = torch.empty_like(g)
        G.shard_reduce_mean_f32(plan, r, [compact_from_flat(plan, f, r) for f in dev],
                                G.LAYOUT_SHARD_COMPACT, gc)
        torch.cuda.synchronize()
        want = reduce_mean([opack.owner_view(oplan, o, r) for o in ref], r)
        assert_bits(host(g), want, f"{w.name}: fp32-contribution mean, owner {r}")
        assert_bits(host(gc), want, f"{w.name}: fp32-contribution mean, owner {r} (shard-compact)")
        sq = sqnorm_partial(want)
        assert abs(host(part)[0] - sq) <= 1e-12 * sq


@pytest.mark.parametrize("P", [1, 2, 3, 5, 6, 7, 8, 16, 100, 256])
def test_fp32_reduce_every_rank_count(P):
    """Fixed-P kernels (2, 8, 16) and the generic loop (1, 3, 5, 6, 7, 100, 256)
    with true division where P is not a power of two."""
    rng = np.random.default_rng(300 + P)
    numel = [int(x) for x in rng.integers(1, 5000, 9)]
    plan = G.Plan(numel, 6000, P, 8).upload()
    oplan = make_plan(numel, 6000, P, align=8)
    host_flats, flats = [], []
    for _ in range(P):
        grads = [np.asarray(rng.integers(0, 65536, n), np.uint16) & 0xBFFF for n in numel]
        host_flats.append(opack.pack_f32(oplan, grads))              # oracle side
        f = torch.empty(plan.flat_len, dtype=torch.float32, device="cuda")
        G.bucket_pack_f32(plan, [torch.from_numpy(x.view(np.int16)).cuda().view(torch.uint16)
                                 for x in grads], f)                 # library side
        flats.append(f)
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    part = torch.zeros(1, dtype=torch.float64, device="cuda")
    for r in sorted({0, P // 2, P - 1}):
        g = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
        G.shard_reduce_mean_f32(plan, r, flats, G.LAYOUT_BUCKET_FLAT, g, part, ws)
        torch.cuda.synchronize()
        want = reduce_mean([opack.owner_view(oplan, f, r) for f in host_flats], r)
        assert_bits(host(g), want, f"P={P} owner {r}")


def test_fp32_accumulation_unaligned_sources():
    numel = [1001, 17, 4096]
    plan = G.Plan(numel, 1 << 20, 2).upload()
    oplan = make_plan(numel, 1 << 20, 2)
    base = torch.arange(1, 8000, dtype=torch.int16, device="cuda").view(torch.uint16)
    grads = [base[1:1 + 1001], base[1003:1003 + 17], base[1021:1021 + 4096]]   # odd offsets
    flat = torch.full((plan.flat_len,), 3.0, dtype=torch.float32, device="cuda")
    G.bucket_pack_f32(plan, grads, flat)
    G.bucket_accumulate_f32(plan, grads, flat)
    torch.cuda.synchronize()
    hg = [host(t) for t in grads]
    want = opack.accumulate_f32(oplan, opack.pack_f32(oplan, hg), hg)
    assert_bits(host(flat), want, "unaligned fp32 accumulation")


@pytest.mark.parametrize("P", [3, 6, 12, 24, 64, 96, 100])
def test_bf16_wire_every_kernel_family(P):
    """The bf16-wire reduce at world sizes that run each kernel form: the
    lane-contiguous kernel with compile-time P (3, 6) and its runtime-P loop
    (12), the 16-byte kernel with compile-time P (24, 64, 96) and its runtime-P
    loop (100), both layouts, against the oracle's bf16-wire ring."""
    from oracle.bf16 import narrow
    rng = np.random.default_rng(700 + P)
    numel = [int(x) for x in rng.integers(1, 4000, 7)]
    plan = G.Plan(numel, 6000, P).upload()
    oplan = make_plan(numel, 6000, P)
    flats, dev = [], []
    for q in range(P):
        x = rng.normal(size=sum(numel)) * np.exp2(rng.integers(-10, 11, size=sum(numel)))
        bits = narrow(x.astype(np.float32))
        grads = [bits[s:s + n] for s, n in zip(OI.prefix(numel), numel)]
        flats.append(opack.pack(oplan, grads))
        f = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, [torch.from_numpy(gq.view(np.int16).copy()).view(torch.uint16).cuda()
                             for gq in grads], f)
        dev.append(f)
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    part = torch.zeros(1, dtype=torch.float64, device="cuda")
    for r in sorted({0, P // 2, P - 1}):
        g = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
        G.shard_reduce_mean(plan, r, dev, G.LAYOUT_BUCKET_FLAT, g, part, ws, bf16_wire=True)
        gc = torch.empty_like(g)
        comp = [torch.cat([f[b["base"] + r * b["chunk"]:b["base"] + (r + 1) * b["chunk"]]
                           for b in plan.buckets()]).contiguous() for f in dev]
        G.shard_reduce_mean(plan, r, comp, G.LAYOUT_SHARD_COMPACT, gc, None, None, bf16_wire=True)
        torch.cuda.synchronize()
        want = reduce_mean_bf16_wire([opack.owner_view(oplan, f, r) for f in flats], r)
        assert_bits(host(g), want, f"bf16-wire P={P} owner {r}")
        assert_bits(host(gc), want, f"bf16-wire P={P} owner {r} (shard-compact)")
        sq = sqnorm_partial(want)
        assert abs(host(part)[0] - sq) <= 1e-12 * max(sq, 1e-300)

