"""GPU parity of the bucket-flat accesses on both of their addressing paths.

The lane-contiguous reduce reads bucket-flat contributions, and AdamW writes
its all-gather output, through buffer descriptors based at each tile's first
position, with 32-bit offsets; a plan whose tiles span 2^31 bytes or more of a
flat buffer (buckets of over 2^29 elements) takes 64-bit addresses instead.
The test build's set_flat_wide hook forces that second path on small plans,
so both run here against the oracle: the shard step of every owner (reduce
and AdamW with the all-gather output), the standalone all-gather writer, the
DDP all-reduce (output at flat positions) and the reduce over fp32
contributions, bit-exact, with the norm
partials equal between the two paths (same grouping)."""
import pytest
import torch

import gradient_sync_zero_amd as G
from oracle import pack as opack
from oracle.norm import sqnorm_partial
from oracle.plan import make_plan
from oracle.reduce import reduce_mean
from oracle.step import ddp_step, zero_step_all_owners
from synth import workloads as W
from tests import gpu_inputs as GI
from tests import oracle_inputs as OI
from tests.parity import assert_bits, host
from tests.test_gpu_parity_small import run_gpu_step

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _test_build():
    with G.test_hooks():
        yield
        G.set_flat_wide(False)


def say(*a):
    print(*a, flush=True)


def packed(plan, w):
    flats = []
    for q in range(w.world_size):
        f = torch.full((plan.flat_len,), 0x7777, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, GI.rank_grads_separate(w, q), f)
        flats.append(f)
    return flats


@pytest.mark.parametrize("cfg", [5, 1])
def test_flat_wide_zero_step(cfg):
    w = W.by_id(cfg)
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    say(f"[{w.name}] ZeRO step, bucket-flat, 64-bit and 32-bit offsets")
    flats_dev = packed(plan, w)
    G.set_flat_wide(True)
    wide = run_gpu_step(w, plan, flats_dev)
    G.set_flat_wide(False)
    buf = run_gpu_step(w, plan, flats_dev)
    flats = [OI.rank_flat(oplan, w, q) for q in range(P)]
    th, m, v = OI.full_state(oplan, w)
    ref = zero_step_all_owners(oplan, flats, th, m, v, w.hp)
    for o, name in ((wide, "64-bit"), (buf, "32-bit")):
        assert o["coef"] == ref["coef"], name
        for r in range(P):
            assert_bits(o["g"][r], ref["g"][r], f"{name} g owner {r}")
            assert abs(o["partials"][r] - ref["partials"][r]) <= 1e-12 * ref["partials"][r]
            for key in ("theta", "m", "v"):
                assert_bits(o[key][r], ref[key][r], f"{name} {key} owner {r}")
            assert_bits(o["shard"][r], ref["p"][r], f"{name} bf16 owner {r}")
        assert_bits(o["gathered"], ref["gathered"], f"{name} gathered bf16")
    assert (wide["partials"] == buf["partials"]).all()
    # the standalone all-gather writer on both store paths
    for on in (True, False):
        G.set_flat_wide(on)
        ag = torch.full((plan.flat_len,), 0x7777, dtype=torch.uint16, device="cuda")
        for r in range(P):
            G.allgather_layout_write(plan, r, buf["shards_dev"][r], ag)
        torch.cuda.synchronize()
        assert_bits(host(ag), ref["gathered"], f"standalone all-gather layout, wide={on}")


@pytest.mark.parametrize("cfg", [5, 1])
def test_flat_wide_allreduce(cfg):
    w = W.by_id(cfg)
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    say(f"[{w.name}] DDP all-reduce, 64-bit and 32-bit offsets")
    flats = packed(plan, w)
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    outs = []
    for on in (True, False):
        G.set_flat_wide(on)
        g_flat = torch.full((plan.flat_len,), float("nan"), dtype=torch.float32, device="cuda")
        parts = torch.zeros(P, dtype=torch.float64, device="cuda")
        G.allreduce_mean(plan, flats, g_flat, parts, ws)
        torch.cuda.synchronize()
        outs.append((host(g_flat), host(parts)))
    oflats = [OI.rank_flat(oplan, w, q) for q in range(P)]
    oth, om, ov = OI.full_state(oplan, w)
    d = ddp_step(oplan, oflats, oth, om, ov, w.hp)
    for (g, parts), name in zip(outs, ("64-bit", "32-bit")):
        assert_bits(g, d["g"], f"{name} all-reduce mean")
        for c in range(P):
            want = sqnorm_partial(opack.owner_view(oplan, d["g"], c))
            assert abs(parts[c] - want) <= 1e-12 * want, f"{name} partial {c}"
    assert (outs[0][1] == outs[1][1]).all()


def test_flat_wide_fp32_contributions():
    w = W.tiny()
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    say(f"[{w.name}] fp32-contribution reduce, 64-bit and 32-bit offsets")
    grads = [GI.rank_grads_separate(w, q) for q in range(P)]
    f32s = []
    for q in range(P):
        f = torch.full((plan.flat_len,), float("nan"), dtype=torch.float32, device="cuda")
        G.bucket_pack_f32(plan, grads[q], f)
        G.bucket_accumulate_f32(plan, grads[(q + 1) % P], f)
        f32s.append(f)
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    hgrads = [OI.rank_grads(w, q) for q in range(P)]
    o32 = [opack.accumulate_f32(oplan, opack.pack_f32(oplan, hgrads[q]), hgrads[(q + 1) % P])
           for q in range(P)]
    for r in range(P):
        want = reduce_mean([opack.owner_view(oplan, f, r) for f in o32], r)
        parts = []
        for on in (True, False):
            G.set_flat_wide(on)
            g = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
            part = torch.zeros(1, dtype=torch.float64, device="cuda")
            G.shard_reduce_mean_f32(plan, r, f32s, G.LAYOUT_BUCKET_FLAT, g, part, ws)
            torch.cuda.synchronize()
            assert_bits(host(g), want, f"fp32-contribution mean owner {r}, wide={on}")
            parts.append(host(part)[0])
        assert abs(parts[0] - sqnorm_partial(want)) <= 1e-12 * sqnorm_partial(want)
        assert parts[0] == parts[1]
