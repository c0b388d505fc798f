"""AdamW at the edges of fp32, on the GPU against the oracle, bit for bit:
denormal weights, moments and gradients (they are kept, not flushed, on both
sides), exact zeros of either sign, v = 0 with and without a gradient, the
first step (t = 1) and a late one (t = 10^4, where both bias corrections round
to 1), a clip coefficient of 1, an ordinary one and a denormal one, and values
large enough for g * g to overflow.  Both entry points: the replicated update
(gsz_adamw_step) and the owned-shard update (gsz_shard_adamw_step).

The optimizer is the AdamW that "Distributed Training: Data Parallel, Model
Parallel and FSDP Strategies" (Inside DDP) calls, with the operation order the
oracle states; the page fixes no precision for these cases, so both sides keep
IEEE fp32 with denormals."""
import numpy as np
import pytest
import torch

import gradient_sync_zero_amd as G
from oracle.adamw import adamw
from synth.workloads import AdamWHP
from tests.parity import assert_bits, host

pytestmark = pytest.mark.gpu

N = 1 << 16


def denormals(rng, n):
    bits = rng.integers(1, 1 << 23, n, dtype=np.uint32) | (rng.integers(0, 2, n, dtype=np.uint32) << 31)
    return bits.view(np.float32)


def edge_arrays(seed):
    """theta, m, v, g with blocks of special values (each block 1/8 of N)."""
    rng = np.random.default_rng(seed)
    f = np.float32
    th = rng.normal(0, 0.02, N).astype(f)
    m = rng.normal(0, 1e-4, N).astype(f)
    v = np.abs(rng.normal(0, 1e-6, N)).astype(f)
    g = rng.normal(0, 1e-3, N).astype(f)
    b = N // 8
    th[0:b] = denormals(rng, b)                          # denormal weights
    m[b:2 * b] = denormals(rng, b)                       # denormal first moments
    v[2 * b:3 * b] = np.abs(denormals(rng, b))           # denormal second moments
    g[3 * b:4 * b] = denormals(rng, b)                   # denormal gradients (g*g underflows)
    v[4 * b:5 * b] = 0.0                                 # v = 0 with a gradient
    m[5 * b:6 * b], v[5 * b:6 * b], g[5 * b:6 * b] = 0.0, 0.0, 0.0   # all zero: pure decay
    g[5 * b:5 * b + 8] = -0.0
    th[5 * b + 8:5 * b + 16] = -0.0
    th[5 * b + 16:5 * b + 1024] = denormals(rng, 1008)  # decays to denormals
    m[5 * b + 1024:5 * b + 2048] = denormals(rng, 1024)  # with g = 0: denormal m'
    m[5 * b + 1024:5 * b + 2048] = np.abs(m[5 * b + 1024:5 * b + 2048])
    g[6 * b:6 * b + 64] = np.float32(3e19)               # g*g overflows to inf
    g[6 * b + 64:6 * b + 128] = np.float32(-2e-19)
    th[7 * b:8 * b] = rng.normal(0, 1e3, b).astype(f)    # large weights
    return th, m, v, g


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


@pytest.mark.parametrize("step", [1, 10, 10000])
@pytest.mark.parametrize("coef", [1.0, 0.0345, 1e-40])
def test_adamw_edge_values_match_the_oracle(step, coef):
    th, m, v, g = edge_arrays([step, int(coef * 1e4)])
    hp = AdamWHP(step=step)
    c = np.float32(coef)
    with np.errstate(over="ignore"):           # g * g overflows on purpose
        ref = adamw(th, m, v, g, c, hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, step)
        assert np.isinf(g[N // 8 * 6] * g[N // 8 * 6])
    coef_d = torch.tensor([c], dtype=torch.float32, device="cuda")
    hpc = G.make_hp(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, step)
    # the replicated update
    dth, dm, dv, dg = dev(th), dev(m), dev(v), dev(g)
    out = torch.empty(N, dtype=torch.uint16, device="cuda")
    G.adamw_step(dth, dm, dv, dg, coef_d, hpc, out)
    # the owned-shard update: a one-tensor plan with one rank, shard-layout output
    plan = G.Plan([N], 1 << 40, 1).upload()
    assert plan.shard_len == N
    sth, sm, sv = dev(th), dev(m), dev(v)
    sout = torch.empty(N, dtype=torch.uint16, device="cuda")
    G.shard_adamw_step(plan, 0, sth, sm, sv, dg, coef_d, hpc, None, sout)
    torch.cuda.synchronize()
    for name, a, b in (("theta", dth, sth), ("m", dm, sm), ("v", dv, sv)):
        k = ("theta", "m", "v").index(name)
        assert_bits(host(a), ref[k], f"{name} (replicated), t={step}, coef={coef}")
        assert_bits(host(b), ref[k], f"{name} (shard), t={step}, coef={coef}")
    assert_bits(host(out), ref[3], "bf16 (replicated)")
    assert_bits(host(sout), ref[3], "bf16 (shard)")
    # denormal results are among those compared (nothing was flushed to zero)
    tiny = np.finfo(np.float32).tiny
    for k in (0, 1):
        assert ((ref[k] != 0) & (np.abs(ref[k]) < tiny)).sum() >= 1000
