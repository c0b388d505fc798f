"""Pins for the oracle's gradient accumulation and bf16-wire ring."""
import numpy as np
import pytest
import torch

from oracle import pack as opack
from oracle.bf16 import narrow, widen
from oracle.plan import make_plan
from oracle.reduce import reduce_mean, reduce_mean_bf16_wire, ring_allreduce_sim
from tests.parity import bf16_wire_bound


def bf16_torch_add(a, b):
    ta = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    return (ta + tb).view(torch.int16).numpy().view(np.uint16)


def test_accumulate_matches_torch_bf16_addition():
    """A bf16 .grad += g in torch (the library routine the training loop runs)."""
    rng = np.random.default_rng(1)
    numel = [1000, 37, 4096, 0, 5]
    plan = make_plan(numel, 4000, 4, align=8)
    g1 = [narrow(rng.normal(0, 1e-3, n).astype(np.float32)) for n in numel]
    g2 = [narrow(rng.normal(0, 1e-3, n).astype(np.float32)) for n in numel]
    flat = opack.pack(plan, g1)
    acc = opack.accumulate(plan, flat, g2)
    for t, n in enumerate(numel):
        off = plan.tensor_offset[t]
        assert np.array_equal(acc[off:off + n], bf16_torch_add(g1[t], g2[t]))
    pad = np.ones(plan.flat_len, bool)
    for t, n in enumerate(numel):
        pad[plan.tensor_offset[t]:plan.tensor_offset[t] + n] = False
    assert not acc[pad].any()
    # accumulating into zeros is packing
    assert np.array_equal(opack.accumulate(plan, np.zeros(plan.flat_len, np.uint16), g2),
                          opack.pack(plan, g2))


def test_accumulate_is_exact_on_small_integers():
    numel = [64, 64]
    plan = make_plan(numel, 1 << 20, 2)
    rng = np.random.default_rng(2)
    ints = [rng.integers(-60, 61, (4, n)) for n in numel]         # sums of 4 stay below 2^8
    flat = np.zeros(plan.flat_len, np.uint16)
    for k in range(4):
        flat = opack.accumulate(plan, flat, [narrow(x[k].astype(np.float32)) for x in ints])
    for t, n in enumerate(numel):
        off = plan.tensor_offset[t]
        assert np.array_equal(widen(flat[off:off + n]), ints[t].sum(axis=0).astype(np.float32))


def test_bf16_wire_equals_message_passing_ring():
    rng = np.random.default_rng(3)
    for P in (2, 3, 8):
        numel = [int(x) for x in rng.integers(1, 2000, 5)]
        plan = make_plan(numel, 3000, P, align=4)
        flats = [opack.pack(plan, [narrow((rng.normal(size=n) * np.exp2(rng.integers(-8, 9, n)))
                                          .astype(np.float32)) for n in numel]) for _ in range(P)]
        res, _, _ = ring_allreduce_sim(plan, flats, bf16_partials=True)
        for r in range(P):
            g = reduce_mean_bf16_wire([opack.owner_view(plan, f, r) for f in flats], r)
            assert np.array_equal(g.view(np.uint32), opack.owner_view(plan, res[0], r).view(np.uint32))


def test_bf16_wire_drifts_from_fp32_but_not_on_exact_inputs():
    rng = np.random.default_rng(4)
    P, n = 8, 100000
    c = [narrow(rng.normal(0, 1e-3, n).astype(np.float32)) for _ in range(P)]
    a, b = reduce_mean(c, 0), reduce_mean_bf16_wire(c, 0)
    assert (a != b).mean() > 0.3                      # per-hop rounding changes most sums
    abs_sum = np.sum([np.abs(widen(x)).astype(np.float64) for x in c], axis=0)
    bound = bf16_wire_bound(abs_sum, P)
    err = np.abs(a.astype(np.float64) - b)
    assert (err <= bound * (1 + 1e-12)).all()
    assert err.max() > 0.25 * bound.max()             # and the bound is not vacuous
    ints = [narrow(rng.integers(-15, 16, n).astype(np.float32)) for _ in range(P)]
    assert np.array_equal(reduce_mean(ints, 3), reduce_mean_bf16_wire(ints, 3))
    one = [c[0]]
    assert np.array_equal(reduce_mean_bf16_wire(one, 0), widen(c[0]))


def test_fp32_accumulation_matches_torch():
    """An fp32 accumulation buffer fed bf16 gradients in torch (acc += g.float())."""
    rng = np.random.default_rng(11)
    numel = [1000, 37, 4096, 0, 5]
    plan = make_plan(numel, 4000, 4, align=8)
    micro = [[narrow(rng.normal(0, 1e-3, n).astype(np.float32)) for n in numel] for _ in range(4)]
    flat = opack.pack_f32(plan, micro[0])
    for k in range(1, 4):
        flat = opack.accumulate_f32(plan, flat, micro[k])
    for t, n in enumerate(numel):
        acc = torch.from_numpy(micro[0][t].view(np.int16)).view(torch.bfloat16).float()
        for k in range(1, 4):
            acc += torch.from_numpy(micro[k][t].view(np.int16)).view(torch.bfloat16).float()
        off = plan.tensor_offset[t]
        assert np.array_equal(flat[off:off + n].view(np.uint32), acc.numpy().view(np.uint32))
    pad = np.ones(plan.flat_len, bool)
    for t, n in enumerate(numel):
        pad[plan.tensor_offset[t]:plan.tensor_offset[t] + n] = False
    assert not flat[pad].any()


def test_fp32_accumulation_is_exact_where_bf16_rounds():
    """Integers up to 2^10 in magnitude: four of them sum exactly in fp32, while
    bf16 (8 significant bits) must round some partial sums."""
    numel = [512]
    plan = make_plan(numel, 1 << 20, 2)
    rng = np.random.default_rng(12)
    ints = rng.integers(-1000, 1001, (4, 512))
    micro = [[narrow(x.astype(np.float32))] for x in ints]
    exact_in = [widen(m[0]).astype(np.float64) for m in micro]   # the bf16-rounded inputs
    f32 = opack.pack_f32(plan, micro[0])
    b16 = opack.pack(plan, micro[0])
    for k in range(1, 4):
        f32 = opack.accumulate_f32(plan, f32, micro[k])
        b16 = opack.accumulate(plan, b16, micro[k])
    want = np.sum(exact_in, axis=0)
    off = plan.tensor_offset[0]
    assert np.array_equal(f32[off:off + 512].astype(np.float64), want)
    assert (widen(b16[off:off + 512]).astype(np.float64) != want).any()


@pytest.mark.parametrize("P", [2, 3, 4, 8])
def test_fp32_contributions_equal_message_passing_ring(P):
    rng = np.random.default_rng(20 + P)
    numel = [int(rng.integers(1, 3000)) for _ in range(6)]
    plan = make_plan(numel, 4000, P, align=8)
    flats = []
    for q in range(P):
        f = opack.pack_f32(plan, [narrow(rng.normal(0, 1e-3, n).astype(np.float32)) for n in numel])
        f = opack.accumulate_f32(plan, f, [narrow(rng.normal(0, 1e-3, n).astype(np.float32))
                                           for n in numel])
        flats.append(f)
    results, rs_sent, _ = ring_allreduce_sim(plan, flats)
    M = plan.flat_len * 4
    for r in range(P):
        g = reduce_mean([opack.owner_view(plan, f, r) for f in flats], r)
        assert np.array_equal(g.view(np.uint32), opack.owner_view(plan, results[0], r).view(np.uint32))
        assert rs_sent[r] * P == (P - 1) * M


def test_reduce_takes_only_bf16_bits_or_fp32():
    with pytest.raises(ValueError):
        reduce_mean([np.zeros(4, np.float64)] * 2, 0)
