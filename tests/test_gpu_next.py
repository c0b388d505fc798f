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
from tests.parity import assert_bits, host

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
        u = 2.0 ** -8       # bf16 unit roundoff; see the oracle pin for the bound
        abs_sum = np.sum([np.abs(widen(c)).astype(np.float64) for c in cs], axis=0)
        bound = (P - 1) * u * (1 + u) ** (P - 1) * abs_sum / P
        err = np.abs(fp32 - ref)
        assert (err <= bound * (1 + 1e-6) + 1e-12).all()
        worst = max(worst, float((err / np.maximum(bound, 1e-300)).max()))
        changed += int((err > 0).sum())
        n_all += err.size
    print(f"[{w.name}] bf16 wire vs fp32 accumulation: {changed / n_all:.1%} of elements differ; "
          f"largest difference {worst:.2f} of the rounding bound", flush=True)
