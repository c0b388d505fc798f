"""Several consecutive steps, with a checkpoint in the middle.

Four steps of the 1M-parameter P=4 workload, every owner, with fresh gradients
each step and the bias-correction exponent t = 10, 11, 12, 13.  After the
second step the optimizer state is copied to host memory, dropped from the GPU
and restored into new device buffers (a checkpoint and resume: the shard state
is plain fp32 arrays plus t).  Every step must equal the oracle bit for bit."""
import dataclasses

import numpy as np
import pytest
import torch

import gradient_sync_zero_amd as G
from oracle.plan import make_plan
from oracle.step import zero_step_all_owners
from synth import gen
from synth import workloads as W
from tests import gpu_inputs as GI
from tests import oracle_inputs as OI
from tests.parity import assert_bits, host

pytestmark = pytest.mark.gpu

STEP_RANK = 2000     # generator rank field of rank q's gradients at step k: 2000 + 16k + q


def dev_grads(w, q, k):
    out = []
    for s0, n in zip(GI.prefix(w.numel), w.numel):
        t = torch.empty(n, dtype=torch.uint16, device="cuda")
        if n:
            gen.dev_fill(t, w.cfg_id, W.KIND_GRAD, STEP_RANK + 16 * k + q, s0, w.grad_std,
                         gen.MODE_BF16)
        out.append(t)
    return out


def host_flat(plan, w, q, k):
    from oracle import pack as opack
    flat = gen.host_fill(w.cfg_id, W.KIND_GRAD, STEP_RANK + 16 * k + q, 0, w.n_params,
                         w.grad_std, gen.MODE_BF16)
    return opack.pack(plan, [flat[s0:s0 + n] for s0, n in zip(OI.prefix(w.numel), w.numel)])


def test_four_steps_with_checkpoint_resume():
    w = W.tiny()
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    oplan = make_plan(w.numel, w.bucket_cap_bytes, P)
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
    states = {r: GI.owner_state(plan, w, r) for r in range(P)}
    th, m, v = OI.full_state(oplan, w)
    for k in range(4):
        hp = dataclasses.replace(w.hp, step=10 + k)
        flats = []
        for q in range(P):
            f = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
            G.bucket_pack(plan, dev_grads(w, q, k), f)
            flats.append(f)
        partials = torch.zeros(P, dtype=torch.float64, device="cuda")
        gs = []
        for r in range(P):
            g = torch.empty(plan.shard_len, dtype=torch.float32, device="cuda")
            G.shard_reduce_mean(plan, r, flats, G.LAYOUT_BUCKET_FLAT, g, partials[r:r + 1], ws)
            gs.append(g)
        coef = torch.empty(1, dtype=torch.float32, device="cuda")
        G.clip_coef(partials, hp.max_norm, coef)
        gathered = torch.zeros(plan.flat_len, dtype=torch.uint16, device="cuda")
        for r in range(P):
            G.shard_adamw_step(plan, r, *states[r], gs[r], coef, hp, gathered, None)
        torch.cuda.synchronize()

        ref = zero_step_all_owners(oplan, [host_flat(oplan, w, q, k) for q in range(P)],
                                   th, m, v, hp)
        assert host(coef)[0] == ref["coef"], f"step {k}"
        for r in range(P):
            for i, key in enumerate(("theta", "m", "v")):
                assert_bits(host(states[r][i]), ref[key][r], f"step {k} owner {r} {key}")
        assert_bits(host(gathered), ref["gathered"], f"step {k} bf16 params")
        # carry the oracle's state forward in flat layout
        th, m, v = th.copy(), m.copy(), v.copy()
        for r in range(P):
            for b, bk in enumerate(oplan.buckets):
                s0, e0 = oplan.chunk_range(b, r)
                sl = slice(bk.shard_off, bk.shard_off + bk.chunk)
                th[s0:e0], m[s0:e0], v[s0:e0] = ref["theta"][r][sl], ref["m"][r][sl], ref["v"][r][sl]

        if k == 1:   # checkpoint to host memory and resume into fresh device buffers
            saved = {r: [x.cpu().clone() for x in states[r]] for r in range(P)}
            del states
            torch.cuda.empty_cache()
            states = {r: [x.cuda() for x in saved[r]] for r in range(P)}
