"""GPU parity on the small workloads, every owner simulated: bucket pack,
ring-order reduce-mean (both layouts), squared-norm partials, clip
coefficient, AdamW and the all-gather layout, against the oracle on the same
seeded inputs.  Bars: bit-exact for packed bytes and the reduced gradient,
fp32 state within 2 ulp and bf16 within 1 ulp (measured: 0), norm within 1e-5
relative."""
import numpy as np
import pytest
import torch

import gradient_sync_zero_amd as G
from oracle import pack as opack
from oracle.norm import clip_coef as o_clip, sqnorm_partial, total as o_total
from oracle.plan import make_plan
from oracle.reduce import reduce_mean as o_reduce
from oracle.step import ddp_step, zero_step_all_owners
from synth import workloads as W
from tests import gpu_inputs as GI
from tests import oracle_inputs as OI
from tests.parity import assert_bits, host, max_bf16_ulp, max_ulp

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def run_gpu_step(w, plan, flats_dev, layout=G.LAYOUT_BUCKET_FLAT, compacts=None):
    """All owners: reduce (+partial), clip, AdamW.  Returns host copies."""
    P = w.world_size
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    partials = torch.zeros(P, dtype=torch.float64, device="cuda")
    gs = []
    for r in range(P):
        g = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
        src = flats_dev if layout == G.LAYOUT_BUCKET_FLAT else compacts[r]
        G.shard_reduce_mean(plan, r, src, layout, g, partials[r:r + 1], ws)
        gs.append(g)
    coef = torch.empty(1, dtype=torch.float32, device="cuda")
    norm = torch.empty(1, dtype=torch.float32, device="cuda")
    tot = torch.empty(1, dtype=torch.float64, device="cuda")
    G.clip_coef(partials, w.hp.max_norm, coef, norm, tot)
    gathered = torch.full((plan.flat_len,), 0xFFFF, dtype=torch.uint16, device="cuda")
    outs = []
    for r in range(P):
        th, m, v = GI.owner_state(plan, w, r)
        shard = torch.empty(plan.shard_len, dtype=torch.uint16, device="cuda")
        G.shard_adamw_step(plan, r, th, m, v, gs[r], coef, w.hp, gathered, shard)
        outs.append((th, m, v, shard))
    torch.cuda.synchronize()
    return dict(g=[host(g) for g in gs], partials=host(partials), coef=host(coef)[0],
                norm=host(norm)[0], total=host(tot)[0],
                theta=[host(o[0]) for o in outs], m=[host(o[1]) for o in outs],
                v=[host(o[2]) for o in outs], shard=[host(o[3]) for o in outs],
                gathered=host(gathered), gs_dev=gs, shards_dev=[o[3] for o in outs])


@pytest.mark.parametrize("cfg", [0, 5, 1])
def test_full_step_all_owners(cfg):
    w = W.by_id(cfg)
    say(f"[{w.name}] planning + packing {w.world_size} ranks on GPU")
    plan = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, w.world_size)
    flats_dev = []
    for q in range(w.world_size):
        grads = GI.rank_grads_separate(w, q)
        flat = torch.full((plan.flat_len,), 0x7777, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, grads, flat)
        flats_dev.append(flat)
    torch.cuda.synchronize()
    flats = [OI.rank_flat(oplan, w, q) for q in range(w.world_size)]
    for q in range(w.world_size):
        assert_bits(host(flats_dev[q]), flats[q], f"pack rank {q}")

    say(f"[{w.name}] reduce / clip / AdamW for every owner (bucket-flat layout)")
    out = run_gpu_step(w, plan, flats_dev)
    th, m, v = OI.full_state(oplan, w)
    ref = zero_step_all_owners(oplan, flats, th, m, v, w.hp)
    for r in range(w.world_size):
        assert_bits(out["g"][r], ref["g"][r], f"g owner {r}")
        assert abs(out["partials"][r] - ref["partials"][r]) <= 1e-5 * ref["partials"][r]
    assert abs(out["total"] - ref["total"]) <= 1e-12 * ref["total"]
    assert out["norm"] == ref["norm"] and out["coef"] == ref["coef"], (out["coef"], ref["coef"])
    # the finalize arithmetic itself: the oracle's clip of the GPU's own total
    assert o_clip(float(out["total"]), w.hp.max_norm) == (out["norm"], out["coef"])
    for r in range(w.world_size):
        for key in ("theta", "m", "v"):
            assert max_ulp(out[key][r], ref[key][r]) <= 2, (key, r)
            assert_bits(out[key][r], ref[key][r], f"{key} owner {r}")   # measured: exact
        assert max_bf16_ulp(out["shard"][r], ref["p"][r]) <= 1
        assert_bits(out["shard"][r], ref["p"][r], f"bf16 owner {r}")
    assert_bits(out["gathered"], ref["gathered"], "gathered bf16 (all-gather layout)")

    # ZeRO-1/2 shards concatenated equal the unsharded DDP update
    d = ddp_step(oplan, flats, th, m, v, w.hp)
    for r in range(w.world_size):
        assert_bits(out["theta"][r], opack.owner_view(oplan, d["theta"], r), f"DDP theta {r}")
    assert_bits(out["gathered"], d["p"], "DDP bf16 params")

    say(f"[{w.name}] shard-compact layout gives the same bits")
    compacts = [GI.compact_contribs(plan, w, r) for r in range(w.world_size)]
    out2 = run_gpu_step(w, plan, None, G.LAYOUT_SHARD_COMPACT, compacts)
    for r in range(w.world_size):
        assert_bits(out2["g"][r], out["g"][r], f"compact g owner {r}")
        assert out2["partials"][r] == out["partials"][r]
    assert_bits(out2["gathered"], out["gathered"], "compact gathered")

    say(f"[{w.name}] standalone all-gather writer and squared norm")
    ag = torch.full((plan.flat_len,), 0x7777, dtype=torch.uint16, device="cuda")
    for r in range(w.world_size):
        G.allgather_layout_write(plan, r, out["shards_dev"][r], ag)
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    sq = torch.zeros(w.world_size, dtype=torch.float64, device="cuda")
    for r in range(w.world_size):
        G.shard_grad_sqnorm(out["gs_dev"][r], sq[r:r + 1], ws)
    torch.cuda.synchronize()
    assert_bits(host(ag), ref["gathered"], "standalone all-gather layout")
    for r in range(w.world_size):
        assert abs(host(sq)[r] - ref["partials"][r]) <= 1e-12 * ref["partials"][r]


def test_gradient_mean_equals_full_batch_gradient_on_gpu():
    """Least squares, 64 samples on 4 ranks: the GPU mean of the four shard
    gradients is exactly the full-batch gradient (exact rationals)."""
    from fractions import Fraction
    from oracle import lsq
    from oracle.bf16 import narrow
    X, theta, Y = W.lsq_problem()
    full = lsq.full_batch_grad(X, theta, Y)
    shards = lsq.shard_grads(X, theta, Y, 4)
    plan = G.Plan([4], 1 << 20, 4).upload()
    flats = []
    for gk in shards:
        bits = narrow(np.array([float(f) for f in gk], np.float32)).view(np.int16)
        t = torch.from_numpy(bits.copy()).view(torch.uint16).cuda()
        flat = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, [t], flat)
        flats.append(flat)
    g = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
    G.shard_reduce_mean(plan, 0, flats, G.LAYOUT_BUCKET_FLAT, g)
    got = host(g)
    assert [Fraction(float(x)) for x in got[:4]] == full
    assert not got[4:].any()


def test_clip_kernel_against_oracle_on_given_partials():
    rng = np.random.default_rng(12)
    cases = [rng.uniform(0, 3, 8), rng.uniform(0, 1e-3, 4), np.zeros(8), np.array([0.25]),
             np.array([1.0]), rng.uniform(100, 200, 64), np.array([np.inf, 1.0]),
             np.array([np.nan, 1.0])]
    for parts in cases:
        d = torch.from_numpy(parts.astype(np.float64)).cuda()
        coef = torch.empty(1, dtype=torch.float32, device="cuda")
        norm = torch.empty(1, dtype=torch.float32, device="cuda")
        tot = torch.empty(1, dtype=torch.float64, device="cuda")
        G.clip_coef(d, 1.0, coef, norm, tot)
        T = o_total(parts)
        n32, c32 = o_clip(T, 1.0)
        gt, gn, gc = host(tot)[0], host(norm)[0], host(coef)[0]
        if np.isnan(T):
            assert np.isnan(gt) and np.isnan(gn) and np.isnan(gc)
            continue
        assert gt == T
        assert gn == n32 and gc == c32, (parts, gn, n32, gc, c32)


@pytest.mark.parametrize("P", [1, 2, 3, 5, 6, 12, 16, 24, 32, 64, 96, 100, 256])
def test_reduce_every_rank_count(P):
    """Static-P kernels (2..64) and the dynamic-P kernel (1, 3, 5, 6, 12, 100,
    and 256 = the largest world size, a full pointer table), power-of-two and
    true-division paths, ragged tensor sizes."""
    rng = np.random.default_rng(P)
    numel = [int(x) for x in rng.integers(1, 3000, 9)]
    numel[0] = 0
    plan = G.Plan(numel, 6000, P).upload()
    oplan = make_plan(numel, 6000, P)
    flats, flats_dev = [], []
    for q in range(P):
        x = rng.normal(size=sum(numel)) * np.exp2(rng.integers(-12, 13, size=sum(numel)))
        from oracle.bf16 import narrow
        bits = narrow(x.astype(np.float32))
        pre = OI.prefix(numel)
        grads = [bits[s:s + n] for s, n in zip(pre, numel)]
        flats.append(opack.pack(oplan, grads))
        flat = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
        dev = [torch.from_numpy(gq.view(np.int16).copy()).view(torch.uint16).cuda() for gq in grads]
        G.bucket_pack(plan, dev, flat)
        flats_dev.append(flat)
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    part = torch.zeros(1, dtype=torch.float64, device="cuda")
    for r in sorted({0, P // 2, P - 1}):
        g = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
        G.shard_reduce_mean(plan, r, flats_dev, G.LAYOUT_BUCKET_FLAT, g, part, ws)
        ref = o_reduce([opack.owner_view(oplan, f, r) for f in flats], r)
        assert_bits(host(g), ref, f"P={P} owner {r}")
        assert abs(host(part)[0] - sqnorm_partial(ref)) <= 1e-12 * sqnorm_partial(ref)


@pytest.mark.parametrize("n", [0, 1, 3, 4, 5, 2047, 2048, 2049, 4099, (1 << 20) + 5, 2048 * 1025 + 7])
def test_standalone_norm_any_length(n):
    """Full 2048-element tiles, a ragged last tile (also not a multiple of 4),
    and enough tiles (> 1024) for the two-stage fixed-order sum."""
    from synth import gen
    x = gen.host_fill(W.tiny().cfg_id, W.KIND_MASTER, 900, 0, n, 0.02, gen.MODE_F32)
    g = torch.from_numpy(np.ascontiguousarray(x)).cuda() if n else torch.empty(0, device="cuda")
    ws = torch.zeros(G.workspace_bytes(n) // 8, dtype=torch.float64, device="cuda")
    part = torch.full((1,), 7.0, dtype=torch.float64, device="cuda")
    G.shard_grad_sqnorm(g, part, ws)
    torch.cuda.synchronize()
    want = sqnorm_partial(x)
    got = host(part)[0]
    assert abs(got - want) <= 1e-12 * want if n else got == 0.0, (n, got, want)


def test_edge_plans_on_gpu():
    part = torch.full((1,), 7.0, dtype=torch.float64, device="cuda")
    # no tensors at all: every call is a no-op and the partial is zero
    plan = G.Plan([], 1 << 20, 4).upload()
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    dummy = torch.zeros(8, dtype=torch.uint16, device="cuda")
    G.shard_reduce_mean(plan, 2, [dummy] * 4, G.LAYOUT_SHARD_COMPACT,
                        torch.zeros(8, device="cuda"), part, ws)
    G.bucket_pack(plan, [], dummy)
    torch.cuda.synchronize()
    assert host(part)[0] == 0.0
    # one tensor over the cap, a cap below every tensor, zero-size tensors
    for numel, cap in (([100000], 1000), ([3, 0, 64, 0, 1000, 5], 2), ([0, 0, 16], 1 << 20)):
        plan = G.Plan(numel, cap, 2).upload()
        oplan = make_plan(numel, cap, 2)
        grads = [(torch.arange(1, n + 1, dtype=torch.int32, device="cuda") & 0x7FFF)
                 .to(torch.int16).view(torch.uint16) for n in numel]
        flat = torch.full((plan.flat_len,), 0x7777, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, grads, flat)
        ref = opack.pack(oplan, [(np.arange(1, n + 1) & 0x7FFF).astype(np.uint16) for n in numel])
        torch.cuda.synchronize()
        assert_bits(host(flat), ref, f"pack {numel} cap {cap}")


def test_unaligned_sources_take_the_element_path():
    numel = [1001, 17, 4096]
    plan = G.Plan(numel, 1 << 20, 2).upload()
    oplan = make_plan(numel, 1 << 20, 2)
    base = torch.arange(1, 8000, dtype=torch.int16, device="cuda").view(torch.uint16)
    grads = [base[1:1 + 1001], base[1003:1003 + 17], base[1021:1021 + 4096]]   # odd offsets
    flat = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
    G.bucket_pack(plan, grads, flat)
    ref = opack.pack(oplan, [host(t) for t in grads])
    torch.cuda.synchronize()
    assert_bits(host(flat), ref, "unaligned pack")


def test_non_finite_values_propagate():
    w = W.tiny()
    plan = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, w.world_size)
    flats = [OI.rank_flat(oplan, w, q) for q in range(4)]
    bad = {2: (100, 0x7FC0), 1: (plan.flat_len - 200000, 0x7F80)}   # a NaN and a +inf
    dev = []
    for q in range(4):                       # the GPU side packs with the library's own plan
        f = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, GI.rank_grads_separate(w, q), f)
        dev.append(f)
    for q, (pos, bits) in bad.items():       # the same positions poisoned on both sides
        flats[q][pos] = bits
        dev[q].view(torch.int16)[pos] = np.int16(np.uint16(bits).view(np.int16))
    out = run_gpu_step(w, plan, dev)
    th, m, v = OI.full_state(oplan, w)
    ref = zero_step_all_owners(oplan, flats, th, m, v, w.hp)
    for r in range(4):
        assert_bits(out["g"][r], ref["g"][r], f"g owner {r}")
    assert np.isnan(out["coef"]) and np.isnan(ref["coef"])
    for r in range(4):
        assert_bits(out["theta"][r], ref["theta"][r], f"theta {r}")


def test_errors_are_reported_not_launched():
    w = W.tiny()
    plan = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size)
    g = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
    c = [torch.zeros(plan.shard_len, dtype=torch.uint16, device="cuda")] * 4
    with pytest.raises(G.GszError) as e:
        G.shard_reduce_mean(plan, 0, c, G.LAYOUT_SHARD_COMPACT, g)
    assert e.value.name == "GSZ_ERR_NOT_UPLOADED"
    plan.upload()
    with pytest.raises(G.GszError) as e:
        G.shard_reduce_mean(plan, 4, c, G.LAYOUT_SHARD_COMPACT, g)
    assert e.value.name == "GSZ_ERR_BAD_RANK"
    with pytest.raises(G.GszError) as e:
        G.shard_reduce_mean(plan, 0, c, 7, g)
    assert e.value.name == "GSZ_ERR_INVALID_ARG"
    buf = torch.zeros(plan.shard_len + 8, dtype=torch.uint16, device="cuda")
    with pytest.raises(G.GszError) as e:
        G.shard_reduce_mean(plan, 0, [buf[1:1 + plan.shard_len]] * 4, G.LAYOUT_SHARD_COMPACT, g)
    assert e.value.name == "GSZ_ERR_MISALIGNED"
    small_ws = torch.zeros(4, dtype=torch.float64, device="cuda")
    part = torch.zeros(1, dtype=torch.float64, device="cuda")
    with pytest.raises(G.GszError) as e:
        G.shard_reduce_mean(plan, 0, c, G.LAYOUT_SHARD_COMPACT, g, part, small_ws)
    assert e.value.name == "GSZ_ERR_SIZE"
    short_ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8 - 1, dtype=torch.float64, device="cuda")
    with pytest.raises(G.GszError) as e:
        G.shard_reduce_mean(plan, 0, c, G.LAYOUT_SHARD_COMPACT, g, part, short_ws)
    assert e.value.name == "GSZ_ERR_SIZE"
    with pytest.raises(G.GszError) as e:
        G.shard_grad_sqnorm(g, part, short_ws[:G.workspace_bytes(g.numel()) // 8 - 1])
    assert e.value.name == "GSZ_ERR_SIZE"
    st = [torch.zeros(plan.shard_len, device="cuda") for _ in range(3)]
    coef = torch.ones(1, device="cuda")
    with pytest.raises(G.GszError):
        G.shard_adamw_step(plan, 0, *st, g, coef, w.hp)          # no output buffer
    odd = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size, align=4).upload()
    with pytest.raises(G.GszError) as e:
        G.shard_reduce_mean(odd, 0, c, G.LAYOUT_SHARD_COMPACT, g)
    assert e.value.name == "GSZ_ERR_INVALID_ARG"


def test_bitwise_deterministic_run_to_run():
    w = W.gpt2_small()
    plan = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size).upload()
    comp = GI.compact_contribs(plan, w, 3)
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    res = []
    for _ in range(3):
        g = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
        part = torch.zeros(1, dtype=torch.float64, device="cuda")
        G.shard_reduce_mean(plan, 3, comp, G.LAYOUT_SHARD_COMPACT, g, part, ws)
        th, m, v = GI.owner_state(plan, w, 3)
        coef = torch.full((1,), 0.25, dtype=torch.float32, device="cuda")
        sh = torch.empty(plan.shard_len, dtype=torch.uint16, device="cuda")
        G.shard_adamw_step(plan, 3, th, m, v, g, coef, w.hp, None, sh)
        torch.cuda.synchronize()
        res.append((host(g), host(part)[0], host(th), host(sh)))
    for k in (1, 2):
        assert_bits(res[k][0], res[0][0], "g rerun")
        assert res[k][1] == res[0][1]
        assert_bits(res[k][2], res[0][2], "theta rerun")
        assert_bits(res[k][3], res[0][3], "bf16 rerun")


@pytest.mark.parametrize("seed", range(12))
def test_random_plans_full_step(seed):
    """Seeded random workloads: 1-24 tensors of 0-30000 elements (some empty),
    bucket caps from 1 KB to 200 KB, P = 1..9, align 8 or 64, clipping active
    or not.  Pack, every owner's reduce (both layouts), clip and AdamW against
    the oracle, bit for bit."""
    import dataclasses
    rng = np.random.default_rng(5000 + seed)
    T = int(rng.integers(1, 25))
    numel = [int(x) for x in rng.integers(0, 30001, T)]
    for k in range(T):
        if rng.random() < 0.15:
            numel[k] = 0
    P = int(rng.integers(1, 10))
    cap = int(rng.integers(1000, 200001))
    align = int(rng.choice([8, 64]))
    std = float(rng.choice([1e-3, 0.1]))
    w = W.Workload(cfg_id=7, name=f"random-{seed}",
                   tensors=tuple((f"t{k}", (n,)) for k, n in enumerate(numel)),
                   world_size=P, bucket_cap_bytes=cap, grad_std=std)
    w = dataclasses.replace(w, hp=dataclasses.replace(w.hp, step=int(rng.integers(1, 20))))
    plan = G.Plan(w.numel, cap, P, align).upload()
    oplan = make_plan(w.numel, cap, P, align=align)
    flats_dev = []
    for q in range(P):
        flat = torch.full((plan.flat_len,), 0x7777, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, GI.rank_grads_separate(w, q), flat)
        flats_dev.append(flat)
    torch.cuda.synchronize()
    flats = [OI.rank_flat(oplan, w, q) for q in range(P)]
    for q in range(P):
        assert_bits(host(flats_dev[q]), flats[q], f"{w.name}: pack rank {q}")
    out = run_gpu_step(w, plan, flats_dev)
    th, m, v = OI.full_state(oplan, w)
    ref = zero_step_all_owners(oplan, flats, th, m, v, w.hp)
    assert out["coef"] == ref["coef"], (out["coef"], ref["coef"])
    for r in range(P):
        assert_bits(out["g"][r], ref["g"][r], f"{w.name}: g owner {r}")
        for key in ("theta", "m", "v"):
            assert_bits(out[key][r], ref[key][r], f"{w.name}: {key} owner {r}")
        assert_bits(out["shard"][r], ref["p"][r], f"{w.name}: bf16 owner {r}")
    assert_bits(out["gathered"], ref["gathered"], f"{w.name}: gathered")
    compacts = [GI.compact_contribs(plan, w, r) for r in range(P)]
    out2 = run_gpu_step(w, plan, None, G.LAYOUT_SHARD_COMPACT, compacts)
    for r in range(P):
        assert_bits(out2["g"][r], out["g"][r], f"{w.name}: compact g owner {r}")


def test_binding_refuses_short_device_buffers():
    """Buffers shorter than the plan implies are refused by the binding before
    any launch (the library sees bare pointers); the right lengths then run."""
    w = W.tiny()
    plan = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size).upload()
    S, L, P = plan.shard_len, plan.flat_len, plan.world_size
    def dev(n, dt=torch.float32):
        if dt == torch.uint16:                   # bf16 bits, made through int16
            return torch.zeros(n, dtype=torch.int16, device="cuda").view(torch.uint16)
        return torch.zeros(n, dtype=dt, device="cuda")
    grads = [dev(n, torch.uint16) for n in w.numel]
    with pytest.raises(ValueError, match="elements"):
        G.bucket_pack(plan, grads, dev(L - 8, torch.uint16))
    with pytest.raises(ValueError, match="elements"):
        G.shard_reduce_mean(plan, 0, [dev(S, torch.uint16)] * (P - 1) + [dev(S - 8, torch.uint16)],
                            G.LAYOUT_SHARD_COMPACT, dev(S))
    with pytest.raises(ValueError, match="elements"):
        G.shard_adamw_step(plan, 0, dev(S), dev(S), dev(S - 4), dev(S), dev(1), w.hp,
                           dev(L, torch.uint16))
    torch.cuda.synchronize()
    flat = dev(L, torch.uint16)
    G.bucket_pack(plan, grads, flat)
    g = dev(S)
    G.shard_reduce_mean(plan, 0, [dev(S, torch.uint16)] * P, G.LAYOUT_SHARD_COMPACT, g)
    torch.cuda.synchronize()
    assert not host(g).any() and not host(flat).any()
