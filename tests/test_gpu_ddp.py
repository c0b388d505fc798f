"""GPU parity of the unshard side and the unsharded (DDP / NO_SHARD) step:
the all-reduce mean against the oracle's message-passing ring, the replicated
AdamW and the unpack into per-parameter tensors against oracle.step.ddp_step
and oracle.pack.unpack, and DDP against the concatenated ZeRO shards -- all bit
for bit."""
import numpy as np
import pytest
import torch

import gradient_sync_zero_amd as G
from oracle import pack as opack
from oracle.norm import sqnorm_partial
from oracle.plan import make_plan
from oracle.step import ddp_step
from synth import workloads as W
from tests import gpu_inputs as GI
from tests import oracle_inputs as OI
from tests.parity import assert_bits, host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("cfg", [0, 5, 1])
def test_ddp_step_and_unpack(cfg):
    w = W.by_id(cfg)
    P = w.world_size
    say(f"[{w.name}] DDP step on GPU")
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    flats = []
    for q in range(P):
        flat = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, GI.rank_grads_separate(w, q), flat)
        flats.append(flat)
    g_flat = torch.full((plan.flat_len,), float("nan"), dtype=torch.float32, device="cuda")
    G.allreduce_mean(plan, flats, g_flat)
    ws = torch.zeros(G.workspace_bytes(plan.flat_len) // 8, dtype=torch.float64, device="cuda")
    part = torch.zeros(1, dtype=torch.float64, device="cuda")
    G.shard_grad_sqnorm(g_flat, part, ws)
    coef = torch.empty(1, dtype=torch.float32, device="cuda")
    tot = torch.empty(1, dtype=torch.float64, device="cuda")
    G.clip_coef(part, w.hp.max_norm, coef, None, tot)
    th, m, v = GI.full_state(plan, w)
    params_flat = torch.full((plan.flat_len,), 0x7777, dtype=torch.uint16, device="cuda")
    G.adamw_step(th, m, v, g_flat, coef, w.hp, params_flat)
    params = [torch.full((n,), 0x7777, dtype=torch.uint16, device="cuda") for n in w.numel]
    G.bucket_unpack(plan, params_flat, params)
    torch.cuda.synchronize()

    oflats = [OI.rank_flat(oplan, w, q) for q in range(P)]
    oth, om, ov = OI.full_state(oplan, w)
    d = ddp_step(oplan, oflats, oth, om, ov, w.hp)
    assert_bits(host(g_flat), d["g"], "all-reduce mean (vs message-passing ring)")
    assert abs(float(host(tot)[0]) - d["total"]) <= 1e-12 * d["total"]
    assert host(coef)[0] == d["coef"]
    assert_bits(host(th), d["theta"], "master")
    assert_bits(host(m), d["m"], "m")
    assert_bits(host(v), d["v"], "v")
    assert_bits(host(params_flat), d["p"], "bf16 params (flat)")
    for t, (a, b) in enumerate(zip(params, opack.unpack(oplan, d["p"]))):
        assert_bits(host(a), b, f"unpacked parameter {t}")

    say(f"[{w.name}] all-reduce with the norm partials fused in")
    g2 = torch.full((plan.flat_len,), float("nan"), dtype=torch.float32, device="cuda")
    parts = torch.full((P,), 7.0, dtype=torch.float64, device="cuda")
    ws2 = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    G.allreduce_mean(plan, flats, g2, parts, ws2)
    coef2 = torch.empty(1, dtype=torch.float32, device="cuda")
    tot2 = torch.empty(1, dtype=torch.float64, device="cuda")
    G.clip_coef(parts, w.hp.max_norm, coef2, None, tot2)
    torch.cuda.synchronize()
    assert_bits(host(g2), d["g"], "all-reduce mean with fused norm")
    hp_ = host(parts)
    for c in range(P):                # partial c is owner c's part of the norm
        want = sqnorm_partial(opack.owner_view(oplan, d["g"], c))
        assert abs(hp_[c] - want) <= 1e-12 * max(want, 1e-300)
    assert abs(float(host(tot2)[0]) - d["total"]) <= 1e-12 * d["total"]
    assert host(coef2)[0] == d["coef"]

    say(f"[{w.name}] DDP chunks equal the ZeRO owners' reduce")
    gf = host(g_flat)
    for r in range(P):
        gr = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
        G.shard_reduce_mean(plan, r, flats, G.LAYOUT_BUCKET_FLAT, gr)
        torch.cuda.synchronize()
        assert_bits(host(gr), opack.owner_view(oplan, gf, r), f"owner {r}")


def test_pack_unpack_round_trip_unaligned():
    w = W.tiny()
    plan = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size).upload()
    grads = GI.rank_grads_separate(w, 2)
    base = torch.zeros(w.n_params + 64, dtype=torch.uint16, device="cuda")
    outs, o = [], 3                       # odd element offsets: unaligned destinations
    for n in w.numel:
        outs.append(base[o:o + n])
        o += n
    flat = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
    G.bucket_pack(plan, grads, flat)
    G.bucket_unpack(plan, flat, outs)
    torch.cuda.synchronize()
    for t, (a, b) in enumerate(zip(outs, grads)):
        assert_bits(host(a), host(b), f"round trip tensor {t}")
    assert not host(base[:3]).any() and not host(base[o:]).any()


def test_adamw_step_rejects_ragged_sizes():
    x = torch.zeros(12, dtype=torch.float32, device="cuda")
    out = torch.zeros(12, dtype=torch.uint16, device="cuda")
    coef = torch.ones(1, device="cuda")
    with pytest.raises(G.GszError) as e:
        G.adamw_step(x, x.clone(), x.clone(), x.clone(), coef, W.AdamWHP(), out)
    assert e.value.name == "GSZ_ERR_SIZE"


@pytest.mark.parametrize("P", [3, 6, 12, 24, 32, 96])
def test_allreduce_every_kernel_family(P):
    """The all-reduce at world sizes that run each kernel form: the
    lane-contiguous kernel with compile-time P (3, 6) and its runtime-P loop
    (12), the 16-byte kernel with compile-time P (24, 32, 96), against the
    message-passing ring, with the chunk owners' norm partials."""
    from oracle.bf16 import narrow
    from oracle.reduce import ring_allreduce_sim
    rng = np.random.default_rng(900 + P)
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
    g = torch.full((plan.flat_len,), float("nan"), dtype=torch.float32, device="cuda")
    parts = torch.zeros(P, dtype=torch.float64, device="cuda")
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    G.allreduce_mean(plan, dev, g, parts, ws)
    torch.cuda.synchronize()
    results, _, _ = ring_allreduce_sim(oplan, flats)
    assert_bits(host(g), results[0], f"all-reduce mean, P={P}")
    for c in range(P):
        want = sqnorm_partial(opack.owner_view(oplan, results[0], c))
        assert abs(host(parts)[c] - want) <= 1e-12 * max(want, 1e-300), (P, c)

