"""Pins for the oracle's bucket plan and pack: invariants that the bucket
rules imply, a brute-force example worked by hand, and closed forms."""
import numpy as np
import pytest

from oracle import pack as opack
from oracle.plan import make_plan
from synth import workloads as W


def check_invariants(plan, cap, P, align=64):
    T = len(plan.numel)
    order = [t for bk in plan.buckets for t in bk.tensors]
    assert order == list(reversed(range(T)))               # reverse order, each tensor once
    base = shard = 0
    for i, bk in enumerate(plan.buckets):
        assert bk.base == base and bk.shard_off == shard
        n = sum(plan.numel[t] for t in bk.tensors)
        assert bk.n == n
        if i < len(plan.buckets) - 1:
            assert 2 * n >= cap                             # closed because it reached the cap
            assert 2 * (n - plan.numel[bk.tensors[-1]]) < cap   # and not before
        assert bk.padded % (P * align) == 0 and 0 <= bk.padded - n < P * align
        assert bk.chunk * P == bk.padded
        pos = bk.base
        for t in bk.tensors:
            assert plan.tensor_offset[t] == pos and plan.tensor_bucket[t] == i
            pos += plan.numel[t]
        base += bk.padded
        shard += bk.chunk
    assert plan.flat_len == base and plan.shard_len == shard and shard * P == base


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_workload_plans_satisfy_invariants(cfg):
    w = W.by_id(cfg)
    plan = make_plan(w.numel, w.bucket_cap_bytes, w.world_size)
    check_invariants(plan, w.bucket_cap_bytes, w.world_size)


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_unpadded_workloads_shard_closed_form(cfg):
    # Every tensor of these models is a multiple of P*64 elements, so no bucket
    # is padded and each shard is exactly Psi/P.
    w = W.by_id(cfg)
    plan = make_plan(w.numel, w.bucket_cap_bytes, w.world_size)
    assert all(bk.padded == bk.n for bk in plan.buckets)
    assert plan.shard_len * w.world_size == w.n_params
    assert plan.shard_len == {2: 163_897_856, 3: 842_301_952, 4: 1_077_760_128}[cfg]


def test_hand_worked_plan():
    # sizes [3,5,2,7], cap 16 bytes (8 bf16), P=2, align=2 (granule 4):
    # reverse order 3 (7 el, 14 B < 16), +2 (9 el, 18 B >= 16: close) ; 1 (5), +0 (8 el = 16 B: close)
    plan = make_plan([3, 5, 2, 7], 16, 2, align=2)
    assert [bk.tensors for bk in plan.buckets] == [(3, 2), (1, 0)]
    assert [(bk.base, bk.n, bk.padded, bk.chunk, bk.shard_off) for bk in plan.buckets] == \
        [(0, 9, 12, 6, 0), (12, 8, 8, 4, 6)]
    assert plan.tensor_offset == (17, 12, 7, 0)
    assert plan.flat_len == 20 and plan.shard_len == 10
    assert plan.chunk_range(0, 1) == (6, 12) and plan.chunk_range(1, 1) == (16, 20)


def test_edge_plans():
    assert make_plan([], 100, 4).buckets == ()
    p = make_plan([1000], 16, 4)                   # one tensor far over the cap sits alone
    assert len(p.buckets) == 1 and p.buckets[0].padded == 1024
    p = make_plan([0, 5, 0], 1 << 20, 2, align=1)  # empty tensors still get a place
    assert p.buckets[0].tensors == (2, 1, 0) and p.buckets[0].n == 5 and p.buckets[0].padded == 6
    p = make_plan([0], 100, 3)
    assert p.flat_len == 0 and p.shard_len == 0
    p = make_plan([7, 9], 10 ** 9, 1)              # P = 1: the shard is the whole (padded) buffer
    assert p.shard_len == p.flat_len == 64
    with pytest.raises(ValueError):
        make_plan([1], 100, 0)


def test_pack_unpack_identity_and_zero_pads():
    w = W.tiny()
    plan = make_plan(w.numel, w.bucket_cap_bytes, w.world_size)
    rng = np.random.default_rng(3)
    grads = [rng.integers(1, 65535, n, dtype=np.uint16) for n in w.numel]
    flat = opack.pack(plan, grads)
    for a, b in zip(opack.unpack(plan, flat), grads):
        assert np.array_equal(a, b)
    mask = np.zeros(plan.flat_len, bool)
    for t, n in enumerate(w.numel):
        mask[plan.tensor_offset[t]:plan.tensor_offset[t] + n] = True
    assert (flat[~mask] == 0).all() and (flat[mask] != 0).all()
    # the owners' views interleave back into the flat buffer
    rebuilt = np.zeros_like(flat)
    for r in range(plan.world_size):
        view = opack.owner_view(plan, flat, r)
        assert view.size == plan.shard_len
        for b, bk in enumerate(plan.buckets):
            s, e = plan.chunk_range(b, r)
            rebuilt[s:e] = view[bk.shard_off:bk.shard_off + bk.chunk]
    assert np.array_equal(rebuilt, flat)
