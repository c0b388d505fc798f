"""GPU parity of the striding path: every data-sized launch capped at a few
blocks (gsz_test_set_grid_limit, a hook of the test build), so each block walks many tiles -- the path that
uncapped launches take only past 2^31 work-items per launch.  Every row of the
step and the rows beyond it against the oracle: bit-exact bytes and reduced
gradients and state, norm partials within 1e-12 relative (their grouping follows
the grid)."""
import numpy as np
import pytest
import torch

import gradient_sync_zero_amd as G
from oracle import pack as opack
from oracle.norm import sqnorm_partial
from oracle.plan import make_plan
from oracle.reduce import reduce_mean, reduce_mean_bf16_wire
from oracle.step import ddp_step, zero_step_all_owners
from synth import workloads as W
from tests import gpu_inputs as GI
from tests import oracle_inputs as OI
from tests.parity import assert_bits, host
from tests.test_gpu_parity_small import run_gpu_step

pytestmark = pytest.mark.gpu

LIMITS = [1, 3, 8, 100]


@pytest.fixture(autouse=True)
def _test_build():
    """Every call of these tests goes to the test build of the library (the
    same sources with the grid-cap hook), plans included."""
    with G.test_hooks():
        yield
        G.set_grid_limit(0)


def say(*a):
    print(*a, flush=True)


def packed(plan, w):
    flats = []
    for q in range(w.world_size):
        f = torch.full((plan.flat_len,), 0x7777, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, GI.rank_grads_separate(w, q), f)
        flats.append(f)
    return flats


@pytest.mark.parametrize("limit", LIMITS)
def test_strided_zero_step(limit):
    w = W.tiny_clip()
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    say(f"[{w.name}] ZeRO step, grids capped at {limit} blocks")
    G.set_grid_limit(limit)
    flats_dev = packed(plan, w)
    out = run_gpu_step(w, plan, flats_dev)
    compacts = [GI.compact_contribs(plan, w, r) for r in range(P)]
    out2 = run_gpu_step(w, plan, None, G.LAYOUT_SHARD_COMPACT, compacts)
    ag = torch.full((plan.flat_len,), 0x7777, dtype=torch.uint16, device="cuda")
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    sq = torch.zeros(P, dtype=torch.float64, device="cuda")
    for r in range(P):
        G.allgather_layout_write(plan, r, out["shards_dev"][r], ag)
        G.shard_grad_sqnorm(out["gs_dev"][r], sq[r:r + 1], ws)
    torch.cuda.synchronize()

    flats = [OI.rank_flat(oplan, w, q) for q in range(P)]
    for q in range(P):
        assert_bits(host(flats_dev[q]), flats[q], f"pack rank {q}")
    th, m, v = OI.full_state(oplan, w)
    ref = zero_step_all_owners(oplan, flats, th, m, v, w.hp)
    assert out["coef"] == ref["coef"] and ref["coef"] < 1.0
    for o in (out, out2):
        for r in range(P):
            assert_bits(o["g"][r], ref["g"][r], f"g owner {r}")
            assert abs(o["partials"][r] - ref["partials"][r]) <= 1e-12 * ref["partials"][r]
            for key in ("theta", "m", "v"):
                assert_bits(o[key][r], ref[key][r], f"{key} owner {r}")
            assert_bits(o["shard"][r], ref["p"][r], f"bf16 owner {r}")
        assert_bits(o["gathered"], ref["gathered"], "gathered bf16")
    assert_bits(host(ag), ref["gathered"], "standalone all-gather layout")
    for r in range(P):
        assert abs(host(sq)[r] - ref["partials"][r]) <= 1e-12 * ref["partials"][r]


@pytest.mark.parametrize("limit", [1, 7])
def test_strided_ddp_step(limit):
    w = W.tiny_clip()
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    say(f"[{w.name}] DDP step, grids capped at {limit} blocks")
    G.set_grid_limit(limit)
    flats = packed(plan, w)
    g_flat = torch.full((plan.flat_len,), float("nan"), dtype=torch.float32, device="cuda")
    parts = torch.zeros(P, dtype=torch.float64, device="cuda")
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    G.allreduce_mean(plan, flats, g_flat, parts, ws)
    coef = torch.empty(1, dtype=torch.float32, device="cuda")
    tot = torch.empty(1, dtype=torch.float64, device="cuda")
    G.clip_coef(parts, w.hp.max_norm, coef, None, tot)
    th, m, v = GI.full_state(plan, w)
    params_flat = torch.full((plan.flat_len,), 0x7777, dtype=torch.uint16, device="cuda")
    G.adamw_step(th, m, v, g_flat, coef, w.hp, params_flat)
    params = [torch.full((n,), 0x7777, dtype=torch.uint16, device="cuda") for n in w.numel]
    G.bucket_unpack(plan, params_flat, params)
    torch.cuda.synchronize()

    oflats = [OI.rank_flat(oplan, w, q) for q in range(P)]
    oth, om, ov = OI.full_state(oplan, w)
    d = ddp_step(oplan, oflats, oth, om, ov, w.hp)
    assert_bits(host(g_flat), d["g"], "all-reduce mean")
    assert abs(float(host(tot)[0]) - d["total"]) <= 1e-12 * d["total"]
    assert host(coef)[0] == d["coef"]
    assert_bits(host(th), d["theta"], "master")
    assert_bits(host(m), d["m"], "m")
    assert_bits(host(v), d["v"], "v")
    assert_bits(host(params_flat), d["p"], "bf16 params (flat)")
    for t, (a, b) in enumerate(zip(params, opack.unpack(oplan, d["p"]))):
        assert_bits(host(a), b, f"unpacked parameter {t}")


@pytest.mark.parametrize("limit", [1, 5])
def test_strided_accumulation_and_reduce_variants(limit):
    w = W.tiny()
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    say(f"[{w.name}] accumulation, fp32 and bf16-wire reduce, grids capped at {limit} blocks")
    G.set_grid_limit(limit)
    grads = [GI.rank_grads_separate(w, q) for q in range(P)]
    hgrads = [OI.rank_grads(w, q) for q in range(P)]
    f16 = torch.full((plan.flat_len,), 0x7777, dtype=torch.uint16, device="cuda")
    G.bucket_pack(plan, grads[0], f16)
    G.bucket_accumulate(plan, grads[1], f16)
    f32s = []
    for q in range(P):
        f = torch.full((plan.flat_len,), float("nan"), dtype=torch.float32, device="cuda")
        G.bucket_pack_f32(plan, grads[q], f)
        G.bucket_accumulate_f32(plan, grads[(q + 1) % P], f)
        f32s.append(f)
    flats = packed(plan, w)
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    part32 = torch.zeros(P, dtype=torch.float64, device="cuda")
    part16 = torch.zeros(P, dtype=torch.float64, device="cuda")
    g32, g16 = [], []
    for r in range(P):
        a = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
        G.shard_reduce_mean_f32(plan, r, f32s, G.LAYOUT_BUCKET_FLAT, a, part32[r:r + 1], ws)
        b = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
        G.shard_reduce_mean(plan, r, flats, G.LAYOUT_BUCKET_FLAT, b, part16[r:r + 1], ws,
                            bf16_wire=True)
        g32.append(a)
        g16.append(b)
    torch.cuda.synchronize()

    want16 = opack.accumulate(oplan, opack.pack(oplan, hgrads[0]), hgrads[1])
    assert_bits(host(f16), want16, "bf16 accumulation")
    o32 = [opack.accumulate_f32(oplan, opack.pack_f32(oplan, hgrads[q]), hgrads[(q + 1) % P])
           for q in range(P)]
    for q in range(P):
        assert_bits(host(f32s[q]), o32[q], f"fp32 accumulation rank {q}")
    oflats = [OI.rank_flat(oplan, w, q) for q in range(P)]
    for r in range(P):
        want = reduce_mean([opack.owner_view(oplan, f, r) for f in o32], r)
        assert_bits(host(g32[r]), want, f"fp32-contribution mean owner {r}")
        assert abs(host(part32)[r] - sqnorm_partial(want)) <= 1e-12 * sqnorm_partial(want)
        want = reduce_mean_bf16_wire([opack.owner_view(oplan, f, r) for f in oflats], r)
        assert_bits(host(g16[r]), want, f"bf16-wire mean owner {r}")
        assert abs(host(part16)[r] - sqnorm_partial(want)) <= 1e-12 * sqnorm_partial(want)


def test_strided_pack_unaligned_and_ragged():
    """Unaligned tensors and ragged tails take the element paths of the pack
    kernels; under a cap of 2 blocks those run strided too."""
    numel = [1001, 17, 4096, 0, 513, 7]
    plan = G.Plan(numel, 6000, 2).upload()
    oplan = make_plan(numel, 6000, 2)
    G.set_grid_limit(2)
    base = torch.arange(1, 12000, dtype=torch.int16, device="cuda").view(torch.uint16)
    offs = np.cumsum([1] + [n + 1 for n in numel[:-1]])           # every tensor at an odd offset
    grads = [base[o:o + n] for o, n in zip(offs, numel)]
    flat = torch.full((plan.flat_len,), 0x7777, dtype=torch.uint16, device="cuda")
    G.bucket_pack(plan, grads, flat)
    f32 = torch.full((plan.flat_len,), 3.0, dtype=torch.float32, device="cuda")
    G.bucket_pack_f32(plan, grads, f32)
    G.bucket_accumulate_f32(plan, grads, f32)
    outs = [torch.full((n,), 0x7777, dtype=torch.uint16, device="cuda") for n in numel]
    G.bucket_unpack(plan, flat, outs)
    torch.cuda.synchronize()
    hg = [host(t) for t in grads]
    ref = opack.pack(oplan, hg)
    assert_bits(host(flat), ref, "strided pack, unaligned")
    assert_bits(host(f32), opack.accumulate_f32(oplan, opack.pack_f32(oplan, hg), hg),
                "strided fp32 accumulation, unaligned")
    for t, (a, b) in enumerate(zip(outs, opack.unpack(oplan, ref))):
        assert_bits(host(a), b, f"strided unpack tensor {t}")
