"""Pins for the oracle's ring-order mean: the message-passing ring (the order
emerges from the protocol, it is not retyped), exact rational means on dyadic
inputs, the closed-form byte counts the pages derive, and average-not-sum."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import pack as opack
from oracle.bf16 import narrow, widen
from oracle.plan import make_plan
from oracle.reduce import central_gather_sim, reduce_mean, ring_allreduce_sim


def wide_range_bf16(rng, n):
    """bf16 values whose magnitudes span 2^-12..2^12, so rounding order matters."""
    x = rng.normal(size=n) * np.exp2(rng.integers(-12, 13, size=n))
    return narrow(x.astype(np.float32))


@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 8])
def test_direct_mean_equals_message_passing_ring(P):
    rng = np.random.default_rng(P)
    numel = [int(rng.integers(1, 3000)) for _ in range(7)]
    plan = make_plan(numel, 4000, P, align=4)
    flats = [opack.pack(plan, [wide_range_bf16(rng, n) for n in numel]) for _ in range(P)]
    results, rs_sent, ag_sent = ring_allreduce_sim(plan, flats)
    for k in range(1, P):                       # replica invariant: identical bits everywhere
        assert np.array_equal(results[k].view(np.uint32), results[0].view(np.uint32))
    for r in range(P):                          # RS then AG equals the owner's direct mean
        g = reduce_mean([opack.owner_view(plan, f, r) for f in flats], r)
        assert np.array_equal(g.view(np.uint32), opack.owner_view(plan, results[0], r).view(np.uint32))
    M = plan.flat_len * 4                       # bytes of the fp32 tensor being reduced
    for k in range(P):                          # (N-1)/N * M per phase, 2(N-1)/N * M in total
        assert rs_sent[k] * P == (P - 1) * M and ag_sent[k] * P == (P - 1) * M
        assert (rs_sent[k] + ag_sent[k]) * P == 2 * (P - 1) * M


def test_order_matters_so_the_ring_pin_has_teeth():
    rng = np.random.default_rng(7)
    P, n = 8, 20000
    c = [wide_range_bf16(rng, n) for _ in range(P)]
    ring = reduce_mean(c, 0)
    naive = widen(c[0]).copy()
    for q in range(1, P):
        naive = naive + widen(c[q])
    naive = naive / np.float32(P)
    assert (ring.view(np.uint32) != naive.view(np.uint32)).sum() > 0


def test_dyadic_inputs_give_the_exact_rational_mean():
    # integers over 16 with small numerators: every partial sum is exact in fp32
    rng = np.random.default_rng(11)
    for P in (2, 3, 4, 6, 8):
        nums = rng.integers(-96, 97, size=(P, 500))
        c = [narrow((nums[q] / 16.0).astype(np.float32)) for q in range(P)]
        for r in range(P):
            g = reduce_mean(c, r)
            for j in range(0, 500, 37):
                exact = Fraction(int(nums[:, j].sum()), 16 * P)
                assert Fraction(float(g[j])) == exact or P in (3, 6)   # 1/3 is not dyadic
                assert abs(Fraction(float(g[j])) - exact) <= abs(exact) * Fraction(1, 1 << 23)


def test_average_not_sum_and_power_of_two_division():
    rng = np.random.default_rng(5)
    x = narrow(rng.normal(size=4096).astype(np.float32))
    for P in (1, 2, 4, 8, 64):
        g = reduce_mean([x] * P, P - 1)
        assert np.array_equal(g, widen(x))       # P equal gradients average to themselves
    # for P a power of two, sum/P, sum*(1/P) and the sum of c/P agree bit for bit
    c = [wide_range_bf16(rng, 4096) for _ in range(8)]
    acc = widen(c[1]).copy()
    for k in range(2, 9):
        acc = acc + widen(c[k % 8])
    assert np.array_equal(reduce_mean(c, 0), acc * np.float32(0.125))


def test_central_gather_traffic_grows_with_N():
    for P in (2, 4, 8):
        plan = make_plan([256 * P], 1 << 20, P, align=4)
        flats = [np.full(plan.flat_len, 0x3F80, np.uint16)] * P
        res, primary = central_gather_sim(plan, flats)
        assert np.all(res == 1.0)
        assert primary == 2 * (P - 1) * plan.flat_len * 4


def _ring_with_fault(plan, flats, fault):
    """A copy of the message-passing ring with one planted fault (CPU only):
    'drop' loses the first reduce-scatter message of bucket 0; 'dup' delivers it
    twice."""
    P = plan.world_size
    results = [np.zeros(plan.flat_len, dtype=np.float32) for _ in range(P)]
    sent = [0] * P
    for bi, bk in enumerate(plan.buckets):
        C = bk.chunk
        buf = [[widen(flats[k][bk.base + c * C: bk.base + (c + 1) * C]).copy()
                for c in range(P)] for k in range(P)]
        for s in range(P - 1):
            msgs = [(k, (k - 1 - s) % P, buf[k][(k - 1 - s) % P].copy()) for k in range(P)]
            for idx, (k, c, m) in enumerate(msgs):
                first = bi == 0 and s == 0 and idx == 0
                if fault == "drop" and first:
                    continue
                sent[k] += C * 4
                buf[(k + 1) % P][c] = m + buf[(k + 1) % P][c]
                if fault == "dup" and first:
                    sent[k] += C * 4
                    buf[(k + 1) % P][c] = m + buf[(k + 1) % P][c]
        for c in range(P):
            buf[c][c] = (buf[c][c] / np.float32(P)).astype(np.float32)
            results[c][bk.base + c * C: bk.base + (c + 1) * C] = buf[c][c]
    return results, sent


@pytest.mark.parametrize("fault", ["drop", "dup"])
def test_a_lost_or_repeated_message_is_caught(fault):
    rng = np.random.default_rng(9)
    P = 4
    numel = [700, 300, 1200]
    plan = make_plan(numel, 2000, P, align=4)
    flats = [opack.pack(plan, [wide_range_bf16(rng, n) for n in numel]) for _ in range(P)]
    res, sent = _ring_with_fault(plan, flats, fault)
    M = plan.flat_len * 4
    traffic_ok = all(s * P == (P - 1) * M for s in sent)
    mean_ok = all(np.array_equal(
        opack.owner_view(plan, res[r], r),
        reduce_mean([opack.owner_view(plan, f, r) for f in flats], r)) for r in range(P))
    assert not traffic_ok and not mean_ok
