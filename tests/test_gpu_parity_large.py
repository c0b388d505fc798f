"""GPU parity at the full workload sizes (1.3B, 7B share, 70B share), in the
launch configuration the benchmark times, for owners other than 0 (owner 0 is
compared on every element by test_gpu_full_coverage.py) and for the rows
beyond the step.  The oracle recomputes sampled elements one by one (random
indices plus the first and last vectors of every bucket's chunk) from the
same seeded inputs; the squared-norm partial is checked by a property that
holds at any size (it equals the fp64 sum of squares of the produced
gradient)."""
import numpy as np
import pytest
import torch

import gradient_sync_zero_amd as G
from oracle.adamw import adamw as o_adamw
from oracle.plan import make_plan
from oracle.reduce import reduce_mean as o_reduce
from synth import gen
from synth import workloads as W
from tests import gpu_inputs as GI
from tests import oracle_inputs as OI
from tests.parity import assert_bits, host

pytestmark = pytest.mark.gpu

COEF = np.float32(0.0345)       # a clip coefficient chosen by the test (oracle side)


def say(*a):
    print(*a, flush=True)


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def sample_indices(oplan, n_random, seed):
    rng = np.random.default_rng(seed)
    S = oplan.shard_len
    edges = []
    for bk in oplan.buckets:
        if bk.chunk:
            edges += list(range(bk.shard_off, bk.shard_off + 8))
            edges += list(range(bk.shard_off + bk.chunk - 8, bk.shard_off + bk.chunk))
    idx = np.concatenate([rng.integers(0, S, n_random), np.array(edges, np.int64), [0, S - 1]])
    return np.unique(idx)


def gather_dev(t, idx):
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
        return host(t[torch.from_numpy(idx).cuda()].view(torch.uint16))
    return host(t[torch.from_numpy(idx).cuda()])


# Owner 0 is compared on every shard element by test_gpu_full_coverage.py; the
# samples here cover other owners, whose chunks sit elsewhere in every bucket
# and whose rings start elsewhere.
@pytest.mark.parametrize("cfg,layout,owners", [
    (2, G.LAYOUT_BUCKET_FLAT, (3, 7)),
    (3, G.LAYOUT_BUCKET_FLAT, (3, 7)),
    (4, G.LAYOUT_SHARD_COMPACT, (31, 63)),
])
def test_full_size_sampled(cfg, layout, owners):
    w = W.by_id(cfg)
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    assert plan.shard_len == oplan.shard_len
    S = plan.shard_len
    flats = None
    if layout == G.LAYOUT_BUCKET_FLAT:
        say(f"[{w.name}] generating and packing {P} ranks x {w.n_params} gradients")
        buf = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
        flats = []
        for q in range(P):
            _, views = GI.rank_grads(w, q, buf)
            flat = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
            G.bucket_pack(plan, views, flat)
            flats.append(flat)
        torch.cuda.synchronize()
        del buf, views
        # pack parity on sampled flat positions of every rank
        rng = np.random.default_rng(cfg)
        fpos = np.unique(np.concatenate([rng.integers(0, plan.flat_len, 1 << 18),
                                         [0, plan.flat_len - 1]]))
        pidx = OI.param_index_of_flat(oplan, fpos)
        for q in range(P):
            ref = OI.values_at(w, W.KIND_GRAD, q, w.grad_std, gen.MODE_BF16, pidx)
            assert_bits(gather_dev(flats[q], fpos), ref, f"pack rank {q} (sampled)")

    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    for r in owners:
        contribs = flats if flats is not None else None
        if contribs is None:
            say(f"[{w.name}] generating {P} shard-compact contributions for owner {r}")
            contribs = GI.compact_contribs(plan, w, r)
        say(f"[{w.name}] owner {r}: reduce-mean over {P} ranks, S={S}")
        g = torch.empty(S, dtype=torch.float32, device="cuda")
        part = torch.zeros(1, dtype=torch.float64, device="cuda")
        G.shard_reduce_mean(plan, r, contribs, layout, g, part, ws)
        torch.cuda.synchronize()
        if flats is None:
            del contribs
            torch.cuda.empty_cache()

        idx = sample_indices(oplan, 1 << 20, 100 + r)
        fp = OI.flat_pos_of_shard(oplan, r, idx)
        pidx = OI.param_index_of_flat(oplan, fp)
        cs = [OI.values_at(w, W.KIND_GRAD, q, w.grad_std, gen.MODE_BF16, pidx) for q in range(P)]
        g_ref = o_reduce(cs, r)
        assert_bits(gather_dev(g, idx), g_ref, f"g owner {r} (sampled)")

        # property at full size: the partial is the fp64 sum of squares of g
        prop = 0.0
        for c in torch.split(g, 1 << 28):
            prop += float(torch.sum(c.double() * c.double()))
        got = float(host(part)[0])
        assert abs(got - prop) <= 1e-12 * prop, (got, prop)

        say(f"[{w.name}] owner {r}: AdamW with coefficient {COEF}")
        th, m, v = GI.owner_state(plan, w, r)
        coef = torch.full((1,), float(COEF), dtype=torch.float32, device="cuda")
        gathered = shard_out = None
        if layout == G.LAYOUT_BUCKET_FLAT:
            gathered = torch.zeros(plan.flat_len, dtype=torch.uint16, device="cuda")
        else:
            shard_out = torch.zeros(S, dtype=torch.uint16, device="cuda")
        G.shard_adamw_step(plan, r, th, m, v, g, coef, w.hp, gathered, shard_out)
        torch.cuda.synchronize()
        st = [OI.values_at(w, kind, 0, std, mode, pidx) for kind, std, mode in OI.STATE_KINDS]
        hp = w.hp
        t1, m1, v1, p1 = o_adamw(st[0], st[1], st[2], g_ref, COEF, hp.lr, hp.beta1, hp.beta2,
                                 hp.eps, hp.weight_decay, hp.step)
        assert_bits(gather_dev(th, idx), t1, f"master owner {r} (sampled)")
        assert_bits(gather_dev(m, idx), m1, f"m owner {r} (sampled)")
        assert_bits(gather_dev(v, idx), v1, f"v owner {r} (sampled)")
        if gathered is not None:
            assert_bits(gather_dev(gathered, fp), p1, f"bf16 all-gather layout owner {r}")
        else:
            assert_bits(gather_dev(shard_out, idx), p1, f"bf16 shard owner {r}")
        del th, m, v, g, gathered, shard_out
        torch.cuda.empty_cache()


MICRO32 = 3000      # generator rank fields: micro-batch k of rank 0, and fp32 contribution q


def sampled_accumulation(micro, fp32):
    """The oracle's accumulation of the micro-batches' values at sampled
    positions: a one-tensor plan whose elements are the samples (a pad sample
    carries 0 in every micro-batch, which accumulates to the pad's 0)."""
    from oracle import pack as opack
    n = micro[0].size
    plan1 = make_plan([n], 1 << 40, 1, align=1)
    if fp32:
        flat = opack.pack_f32(plan1, [micro[0]])
        for mk in micro[1:]:
            flat = opack.accumulate_f32(plan1, flat, [mk])
    else:
        flat = opack.pack(plan1, [micro[0]])
        for mk in micro[1:]:
            flat = opack.accumulate(plan1, flat, [mk])
    return flat[:n]


def test_fp32_rows_full_size_sampled():
    """The fp32 accumulation buckets and the reduce over fp32 contributions at
    the 7B share's size, in the launch shapes the benchmark times: two
    micro-batches widened and added into rank 0's fp32 buckets (sampled flat
    positions), and the reduce over 8 shard-compact fp32 contributions for
    owner 0 (sampled shard elements; the norm partial by its property)."""
    w = W.by_id(3)
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    S = plan.shard_len

    say(f"[{w.name}] fp32 buckets: widen micro-batch 0, add micro-batch 1")
    buf = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
    flat32 = torch.empty(plan.flat_len, dtype=torch.float32, device="cuda")
    views = [buf[s0:s0 + n] for s0, n in zip(GI.prefix(w.numel), w.numel)]
    for k in (0, 1):
        gen.dev_fill(buf, w.cfg_id, W.KIND_GRAD, MICRO32 + k, 0, w.grad_std, gen.MODE_BF16)
        (G.bucket_pack_f32 if k == 0 else G.bucket_accumulate_f32)(plan, views, flat32)
        torch.cuda.synchronize()                       # buf is refilled for the next micro-batch
    del buf, views
    rng = np.random.default_rng(33)
    fpos = np.unique(np.concatenate([rng.integers(0, plan.flat_len, 1 << 18),
                                     [0, plan.flat_len - 1]]))
    pidx = OI.param_index_of_flat(oplan, fpos)
    mb = [OI.values_at(w, W.KIND_GRAD, MICRO32 + k, w.grad_std, gen.MODE_BF16, pidx)
          for k in (0, 1)]
    assert_bits(gather_dev(flat32, fpos), sampled_accumulation(mb, fp32=True),
                "fp32 buckets (sampled)")
    del flat32
    torch.cuda.empty_cache()

    say(f"[{w.name}] reduce over {P} fp32 shard-compact contributions, S={S}")
    pieces = GI.owner_pieces(plan, w, 0)
    contribs = []
    for q in range(P):
        t = torch.zeros(S, dtype=torch.float32, device="cuda")
        GI.fill_pieces(t, pieces, w, W.KIND_GRAD, MICRO32 + 16 + q, w.grad_std, gen.MODE_F32)
        contribs.append(t)
    g = torch.empty(S, dtype=torch.float32, device="cuda")
    part = torch.zeros(1, dtype=torch.float64, device="cuda")
    ws = torch.zeros(G.workspace_bytes(S) // 8, dtype=torch.float64, device="cuda")
    G.shard_reduce_mean_f32(plan, 0, contribs, G.LAYOUT_SHARD_COMPACT, g, part, ws)
    torch.cuda.synchronize()
    del contribs
    idx = sample_indices(oplan, 1 << 20, 200)
    pidx = OI.param_index_of_flat(oplan, OI.flat_pos_of_shard(oplan, 0, idx))
    cs = [OI.values_at(w, W.KIND_GRAD, MICRO32 + 16 + q, w.grad_std, gen.MODE_F32, pidx)
          for q in range(P)]
    assert_bits(gather_dev(g, idx), o_reduce(cs, 0), "fp32-contribution mean (sampled)")
    prop = 0.0
    for c in torch.split(g, 1 << 28):
        prop += float(torch.sum(c.double() * c.double()))
    got = float(host(part)[0])
    assert abs(got - prop) <= 1e-12 * prop, (got, prop)


def test_bf16_rows_full_size_sampled():
    """The bf16 gradient accumulation and the bf16-wire reduce at the 7B share's
    size, in the launch shapes the benchmark times: micro-batches 0 and 1 into
    rank 0's bf16 buckets (sampled flat positions), and the bf16-wire reduce
    over the 8 ranks' packed buckets for owner 0 (sampled shard elements)."""
    from oracle.reduce import reduce_mean_bf16_wire
    w = W.by_id(3)
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    S = plan.shard_len

    say(f"[{w.name}] bf16 buckets: pack micro-batch 0, accumulate micro-batch 1")
    buf = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
    views = [buf[s0:s0 + n] for s0, n in zip(GI.prefix(w.numel), w.numel)]
    acc = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
    for k in (0, 1):
        gen.dev_fill(buf, w.cfg_id, W.KIND_GRAD, MICRO32 + k, 0, w.grad_std, gen.MODE_BF16)
        (G.bucket_pack if k == 0 else G.bucket_accumulate)(plan, views, acc)
        torch.cuda.synchronize()
    rng = np.random.default_rng(34)
    fpos = np.unique(np.concatenate([rng.integers(0, plan.flat_len, 1 << 18),
                                     [0, plan.flat_len - 1]]))
    pidx = OI.param_index_of_flat(oplan, fpos)
    mb = [OI.values_at(w, W.KIND_GRAD, MICRO32 + k, w.grad_std, gen.MODE_BF16, pidx)
          for k in (0, 1)]
    assert_bits(gather_dev(acc, fpos), sampled_accumulation(mb, fp32=False),
                "bf16 buckets (sampled)")
    del acc

    say(f"[{w.name}] bf16-wire reduce over {P} ranks' buckets, S={S}")
    flats = []
    for q in range(P):
        _, v2 = GI.rank_grads(w, q, buf)
        f = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, v2, f)
        flats.append(f)
    torch.cuda.synchronize()
    del buf, views
    g = torch.empty(S, dtype=torch.float32, device="cuda")
    G.shard_reduce_mean(plan, 0, flats, G.LAYOUT_BUCKET_FLAT, g, bf16_wire=True)
    torch.cuda.synchronize()
    del flats
    idx = sample_indices(oplan, 1 << 20, 300)
    pidx = OI.param_index_of_flat(oplan, OI.flat_pos_of_shard(oplan, 0, idx))
    cs = [OI.values_at(w, W.KIND_GRAD, q, w.grad_std, gen.MODE_BF16, pidx) for q in range(P)]
    assert_bits(gather_dev(g, idx), reduce_mean_bf16_wire(cs, 0), "bf16-wire mean (sampled)")


def test_ddp_full_size_sampled():
    """The unsharded (DDP) step at the 1.3B model's full size, in the launch
    configuration of `bench.py --variant ddp --config 2`: the all-reduce mean
    over the P bucket-flat buffers (each chunk summed in the ring order that
    ends at its owner), the owners' fused norm partials, AdamW over the whole
    flat buffer and the unpack, checked at sampled flat positions against the
    oracle recomputed from the same seeded inputs."""
    w = W.by_id(2)
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    L = plan.flat_len
    say(f"[{w.name}] DDP: generating and packing {P} ranks x {w.n_params} gradients")
    buf = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
    flats = []
    for q in range(P):
        _, views = GI.rank_grads(w, q, buf)
        flat = torch.empty(L, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, views, flat)
        flats.append(flat)
    torch.cuda.synchronize()
    del buf, views
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    parts = torch.zeros(P, dtype=torch.float64, device="cuda")
    g = torch.empty(L, dtype=torch.float32, device="cuda")
    say(f"[{w.name}] DDP: all-reduce mean over {P} ranks, L={L}")
    G.allreduce_mean(plan, flats, g, parts, ws)
    torch.cuda.synchronize()

    # sampled flat positions: random, plus both ends of every chunk of every bucket
    rng = np.random.default_rng(7)
    edges = []
    for bk in oplan.buckets:
        for c in range(P):
            s0 = bk.base + c * bk.chunk
            edges += [s0, s0 + 1, s0 + bk.chunk - 2, s0 + bk.chunk - 1]
    fpos = np.unique(np.concatenate([rng.integers(0, L, 1 << 20), np.array(edges, np.int64)]))
    bases = np.array([bk.base for bk in oplan.buckets], np.int64)
    chunks = np.array([bk.chunk for bk in oplan.buckets], np.int64)
    b = np.searchsorted(bases, fpos, side="right") - 1
    owner = (fpos - bases[b]) // chunks[b]
    pidx = OI.param_index_of_flat(oplan, fpos)
    cs = [OI.values_at(w, W.KIND_GRAD, q, w.grad_std, gen.MODE_BF16, pidx) for q in range(P)]
    g_ref = np.empty(fpos.size, np.float32)
    for c in range(P):
        sel = owner == c
        g_ref[sel] = o_reduce([x[sel] for x in cs], c)
    assert_bits(gather_dev(g, fpos), g_ref, "DDP g (sampled)")

    # property at full size: partials[c] is the fp64 sum of squares of owner c's chunks
    got = host(parts)
    for c in range(P):
        prop = 0.0
        for bk in oplan.buckets:
            x = g[bk.base + c * bk.chunk: bk.base + (c + 1) * bk.chunk].double()
            prop += float(torch.sum(x * x))
        assert abs(got[c] - prop) <= 1e-12 * prop, (c, got[c], prop)

    say(f"[{w.name}] DDP: AdamW over the whole flat buffer with coefficient {COEF}, then unpack")
    del flats, ws
    torch.cuda.empty_cache()
    th, m, v = GI.full_state(plan, w)
    coef = torch.full((1,), float(COEF), dtype=torch.float32, device="cuda")
    pflat = torch.empty(L, dtype=torch.uint16, device="cuda")
    G.adamw_step(th, m, v, g, coef, w.hp, pflat)
    pbuf = torch.empty(w.n_params, dtype=torch.int16, device="cuda").view(torch.uint16)
    pre = GI.prefix(w.numel)
    params = [pbuf[s0:s0 + n] for s0, n in zip(pre, w.numel)]
    G.bucket_unpack(plan, pflat, params)
    torch.cuda.synchronize()
    st = [OI.values_at(w, kind, 0, std, mode, pidx) for kind, std, mode in OI.STATE_KINDS]
    hp = w.hp
    t1, m1, v1, p1 = o_adamw(st[0], st[1], st[2], g_ref, COEF, hp.lr, hp.beta1, hp.beta2,
                             hp.eps, hp.weight_decay, hp.step)
    assert_bits(gather_dev(th, fpos), t1, "DDP master (sampled)")
    assert_bits(gather_dev(m, fpos), m1, "DDP m (sampled)")
    assert_bits(gather_dev(v, fpos), v1, "DDP v (sampled)")
    assert_bits(gather_dev(pflat, fpos), p1, "DDP bf16 flat (sampled)")
    # unpack: parameter index i of a non-pad sample holds the flat value at its position
    real = pidx >= 0
    assert_bits(gather_dev(pbuf, pidx[real]), p1[real], "DDP unpacked parameters (sampled)")
    del th, m, v, g, pflat, pbuf, params
    torch.cuda.empty_cache()
