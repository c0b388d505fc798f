"""GPU parity of the rank-interleaved receive layout (GSZ_LAYOUT_RANK_INTERLEAVED):
one buffer in which rank q's values for shard elements [512t, 512t + 512) sit
at (t*P + q)*512.  The reduce over it must equal the oracle's ring-order mean
bit for bit, like the other layouts, for every world size the kernels
specialise (P <= 16: the lane-contiguous kernel; larger P: the 16-byte one) and
for the runtime-P loops, with ragged last tiles; the bf16-wire and fp32
variants too.  Its fp64 norm partials equal the shard-compact layout's bit for
bit (the same elements per lane, in the same order)."""
import numpy as np
import pytest
import torch

import gradient_sync_zero_amd as G
from oracle.norm import sqnorm_partial
from oracle.plan import make_plan
from oracle.reduce import reduce_mean, reduce_mean_bf16_wire
from synth import workloads as W
from tests import gpu_inputs as GI
from tests import oracle_inputs as OI
from tests.parity import assert_bits, host

pytestmark = pytest.mark.gpu

PIECE = G.INTERLEAVE_PIECE


def say(*a):
    print(*a, flush=True)


def interleave(contribs, P, S, dtype):
    """The interleaved receive buffer of P per-rank shard arrays (host)."""
    T = -(-S // PIECE)
    buf = np.zeros((T, P, PIECE), dtype=dtype)
    for q, c in enumerate(contribs):
        pad = np.zeros(T * PIECE, dtype=dtype)
        pad[:S] = c
        buf[:, q, :] = pad.reshape(T, PIECE)
    return buf.reshape(-1)


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.uint16)
    return torch.from_numpy(a).to("cuda")


def random_bf16(rng, n, std=1e-3):
    x = torch.from_numpy(rng.normal(0, std, n).astype(np.float32)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def reduce_three_ways(plan, P, r, contribs_host, f32=False, wire=False):
    """g and partial from the interleaved and the shard-compact layouts."""
    S = plan.shard_len
    dt = np.float32 if f32 else np.uint16
    ibuf = dev(interleave(contribs_host, P, S, dt))
    assert ibuf.numel() == G.interleaved_len(plan)
    comp = [dev(c) for c in contribs_host]
    ws = torch.zeros(G.workspace_bytes(S) // 8, dtype=torch.float64, device="cuda")
    out = {}
    for name, lay, src in (("ilv", G.LAYOUT_RANK_INTERLEAVED, [ibuf]),
                           ("compact", G.LAYOUT_SHARD_COMPACT, comp)):
        g = torch.full((S,), float("nan"), dtype=torch.float32, device="cuda")
        part = torch.zeros(1, dtype=torch.float64, device="cuda")
        if f32:
            G.shard_reduce_mean_f32(plan, r, src, lay, g, part, ws)
        else:
            G.shard_reduce_mean(plan, r, src, lay, g, part, ws, bf16_wire=wire)
        torch.cuda.synchronize()
        out[name] = (host(g), float(host(part)[0]))
    return out


@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 8, 12, 16, 24, 32, 48, 64, 96, 100, 256])
def test_interleaved_matches_oracle_at_every_world_size(P):
    rng = np.random.default_rng([7, P])
    # one tensor, align 8: S = ceil(n / 8P) * 8 (up to ~40,000: several blocks),
    # a ragged last tile for most P
    n = max(1, int(rng.integers(1, 40000)) * P - int(rng.integers(0, 8 * P)))
    plan = G.Plan([n], 1 << 40, P, 8).upload()
    S = plan.shard_len
    owners = sorted({0, P - 1, int(rng.integers(0, P))})
    say(f"P={P} S={S} (S mod 512 = {S % PIECE}) owners {owners}")
    for r in owners:
        cs = [random_bf16(rng, S) for _ in range(P)]
        out = reduce_three_ways(plan, P, r, cs)
        ref = reduce_mean(cs, r)
        assert_bits(out["ilv"][0], ref, f"interleaved g, P={P} owner {r}")
        assert_bits(out["compact"][0], ref, f"compact g, P={P} owner {r}")
        assert out["ilv"][1] == out["compact"][1], "norm partials differ between layouts"
        want = sqnorm_partial(ref)
        assert abs(out["ilv"][1] - want) <= 1e-12 * max(want, 1e-300)


@pytest.mark.parametrize("P", [3, 8, 64])
def test_interleaved_bf16_wire_and_fp32_rows(P):
    rng = np.random.default_rng([11, P])
    plan = G.Plan([int(rng.integers(20000, 90000))], 1 << 40, P, 8).upload()
    S = plan.shard_len
    r = P // 2
    cs = [random_bf16(rng, S) for _ in range(P)]
    out = reduce_three_ways(plan, P, r, cs, wire=True)
    ref = reduce_mean_bf16_wire(cs, r)
    assert_bits(out["ilv"][0], ref, f"bf16-wire interleaved P={P}")
    assert_bits(out["compact"][0], ref, f"bf16-wire compact P={P}")
    f = [rng.normal(0, 1e-3, S).astype(np.float32) for _ in range(P)]
    out = reduce_three_ways(plan, P, r, f, f32=True)
    ref = reduce_mean(f, r)
    assert_bits(out["ilv"][0], ref, f"fp32 interleaved P={P}")
    assert out["ilv"][1] == out["compact"][1]


@pytest.mark.parametrize("cfg", [0, 1])
def test_interleaved_placement_of_a_workload(cfg):
    """The seeded workload placed by the input module (synth.placement, one
    launch per rank) into the interleaved buffer: the reduce equals the
    oracle's on the oracle's own placement of the same values, every owner."""
    w = W.by_id(cfg)
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    for r in range(P):
        buf = GI.interleaved_contribs(plan, w, r, G.interleaved_len(plan))
        g = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
        part = torch.zeros(1, dtype=torch.float64, device="cuda")
        G.shard_reduce_mean(plan, r, [buf], G.LAYOUT_RANK_INTERLEAVED, g, part, ws)
        torch.cuda.synchronize()
        idx = OI.shard_param_index(oplan, r)
        cs = [OI.values_at(w, W.KIND_GRAD, q, w.grad_std, 2, idx) for q in range(P)]
        ref = reduce_mean(cs, r)
        assert_bits(host(g), ref, f"{w.name} interleaved g owner {r}")
        want = sqnorm_partial(ref)
        assert abs(float(host(part)[0]) - want) <= 1e-12 * want


def test_interleaved_argument_checks():
    P = 4
    plan = G.Plan([5000], 1 << 20, P, 8).upload()
    S = plan.shard_len
    g = torch.empty(S, dtype=torch.float32, device="cuda")
    ok = torch.zeros(G.interleaved_len(plan), dtype=torch.uint16, device="cuda")
    short = torch.zeros(G.interleaved_len(plan) - 8, dtype=torch.uint16, device="cuda")
    with pytest.raises(ValueError):               # one receive buffer, not P
        G.shard_reduce_mean(plan, 0, [ok] * P, G.LAYOUT_RANK_INTERLEAVED, g)
    with pytest.raises(ValueError):               # shorter than P * ceil(S/512) * 512
        G.shard_reduce_mean(plan, 0, [short], G.LAYOUT_RANK_INTERLEAVED, g)
    lib = G.load()
    arr = (G._binding._P * 1)(None)
    rc = lib.gsz_shard_reduce_mean(plan.handle, 0, arr, G.LAYOUT_RANK_INTERLEAVED, g.data_ptr(),
                                   None, None, 0, None)
    assert rc == -1                               # GSZ_ERR_INVALID_ARG: NULL receive buffer
    arr = (G._binding._P * 1)(ok.data_ptr() + 2)
    rc = lib.gsz_shard_reduce_mean(plan.handle, 0, arr, G.LAYOUT_RANK_INTERLEAVED, g.data_ptr(),
                                   None, None, 0, None)
    assert rc == -2                               # GSZ_ERR_MISALIGNED
    G.shard_reduce_mean(plan, 0, [ok], G.LAYOUT_RANK_INTERLEAVED, g)
    torch.cuda.synchronize()
    assert not host(g).any()                      # zeros in, zeros out
