"""GPU parity of the burst reduce (k_reduce_burst): the kernel of the bf16
reduce (fp32 wire) at P > 16 on shards of 2^23 elements or more, which
reduces chunks of 32768 shard elements into LDS and writes g either a chunk at
a time or, on large shards, from per-wave rings inside clock windows common to
the chip.  Every reduce here runs under five write policies (the product's
choice, chunk writes, full rings only, short jittery windows that leave rings
partly held and wrapping, every row at once), which must give the same g and
norm partial bit for bit.  The test build's gsz_test_set_reduce_path sends
small shards (and the bf16 wire) to it, so that every world size the 16-byte kernels specialise
(compile-time P 24, 32, 64, 96; the runtime-P loop at 17, 48, 100, 256, whose
last (P-1) mod 8 contributions go as one group here), every contribution layout, the bf16 wire,
ragged last chunks and rows, shards below one chunk, capped grids (blocks
walking several chunks; XCD classes with no block) and the no-allocation entry
point are compared with the oracle: g bit for bit, the fp64 norm partial within
1e-12 relative (its grouping follows the grid).  g must also equal the
one-tile-per-block kernel's bit for bit.  The product rule (by size) sends the
70B share's reduce here; the full-size tests check that path at its real size."""
import numpy as np
import pytest
import torch

import gradient_sync_zero_amd as G
from oracle import pack as opack
from oracle.bf16 import narrow
from oracle.norm import sqnorm_partial
from oracle.plan import make_plan
from oracle.reduce import reduce_mean, reduce_mean_bf16_wire
from tests import oracle_inputs as OI
from tests.parity import assert_bits, host

pytestmark = pytest.mark.gpu

CHUNK = 32768
PIECE = G.INTERLEAVE_PIECE


@pytest.fixture(autouse=True)
def _burst_path():
    """Every call goes to the test build with the burst kernel forced."""
    with G.test_hooks():
        G.set_reduce_path(G.REDUCE_PATH_BURST)
        try:
            yield
        finally:
            G.set_reduce_path(G.REDUCE_PATH_BY_SIZE)
            G.set_grid_limit(0)
            G.set_burst_window(0, 0)


def say(*a):
    print(*a, flush=True)


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.uint16)
    return torch.from_numpy(a).to("cuda")


def wide_bf16(rng, n):
    """bf16 values over 25 binades (the sums round at every step)."""
    x = rng.normal(size=n) * np.exp2(rng.integers(-12, 13, size=n))
    return narrow(x.astype(np.float32))


def interleave(contribs, P, S):
    T = -(-S // PIECE)
    buf = np.zeros((T, P, PIECE), dtype=np.uint16)
    for q, c in enumerate(contribs):
        pad = np.zeros(T * PIECE, dtype=np.uint16)
        pad[:S] = c
        buf[:, q, :] = pad.reshape(T, PIECE)
    return buf.reshape(-1)


# (period, window) of gsz_test_set_burst_window: the product's choice, chunk
# writes, full rings only, windows of 0.24 us every 0.64 us, every row at once.
WRITES = [(0, 0), (1 << 14, 0), (1 << 20, 1), (64, 24), (1, 1)]


def reduce_once(plan, r, src, layout, S, wire=False):
    g = torch.full((S,), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(G.workspace_bytes(S) // 8, dtype=torch.float64, device="cuda")
    part = torch.zeros(1, dtype=torch.float64, device="cuda")
    G.shard_reduce_mean(plan, r, src, layout, g, part, ws, bf16_wire=wire)
    torch.cuda.synchronize()
    return host(g), float(host(part)[0])


def reduce(plan, r, src, layout, S, wire=False):
    """The reduce under every write policy: the same g and partial bit for bit."""
    out = None
    try:
        for pw in WRITES:
            G.set_burst_window(*pw)
            g, part = reduce_once(plan, r, src, layout, S, wire)
            if out is None:
                out = (g, part)
            else:
                assert_bits(g, out[0], f"g under write policy {pw}")
                assert part == out[1], ("norm partial under write policy", pw, part, out[1])
    finally:
        G.set_burst_window(0, 0)
    return out


def check_partial(got, ref, what):
    want = sqnorm_partial(ref)
    assert abs(got - want) <= 1e-12 * max(want, 1e-300), (what, got, want)


@pytest.mark.parametrize("P", [17, 24, 32, 48, 64, 96, 100, 256])
def test_burst_shard_compact_and_interleaved(P):
    rng = np.random.default_rng([41, P])
    # one tensor, align 8: S = ceil(n / 8P) * 8, 2-4 chunks, ragged last chunk and row
    n = int(rng.integers(2 * CHUNK + 1, 4 * CHUNK)) * P - int(rng.integers(0, 8 * P))
    plan = G.Plan([n], 1 << 40, P, 8).upload()
    S = plan.shard_len
    owners = sorted({0, P - 1, int(rng.integers(0, P))})
    say(f"P={P} S={S} ({S / CHUNK:.2f} chunks, S mod 512 = {S % 512}) owners {owners}")
    for r in owners:
        cs = [wide_bf16(rng, S) for _ in range(P)]
        ref = reduce_mean(cs, r)
        g, part = reduce(plan, r, [dev(c) for c in cs], G.LAYOUT_SHARD_COMPACT, S)
        assert_bits(g, ref, f"burst compact P={P} owner {r}")
        check_partial(part, ref, f"burst compact P={P} owner {r}")
        gi, parti = reduce(plan, r, [dev(interleave(cs, P, S))], G.LAYOUT_RANK_INTERLEAVED, S)
        assert_bits(gi, ref, f"burst interleaved P={P} owner {r}")
        assert parti == part, "norm partials differ between layouts"
    # the one-tile-per-block kernel on the last owner's inputs: the same g
    G.set_reduce_path(G.REDUCE_PATH_TILE)
    gt, partt = reduce(plan, r, [dev(c) for c in cs], G.LAYOUT_SHARD_COMPACT, S)
    assert_bits(gt, g, f"tile vs burst P={P}")
    check_partial(partt, ref, f"tile P={P}")


@pytest.mark.parametrize("P", [24, 33, 64])
def test_burst_bucket_flat(P):
    """Bucket-flat contributions read through the owner's segments: several
    buckets per chunk, chunks that start inside a bucket, ragged tensors."""
    rng = np.random.default_rng([43, P])
    numel = [int(x) for x in rng.integers(1, 9000, 30)]
    target = int(rng.integers(CHUNK + 1, 2 * CHUNK)) * P         # flat length ~ S * P
    while sum(numel) < target:
        numel += [int(x) for x in rng.integers(1, 9000, 30)]
    cap = 2 * target // 11                                       # ~11 buckets
    plan = G.Plan(numel, cap, P).upload()
    oplan = make_plan(numel, cap, P)
    S = plan.shard_len
    say(f"P={P} tensors {len(numel)} buckets {plan.n_buckets} S={S} ({S / CHUNK:.2f} chunks)")
    pre = OI.prefix(numel)
    flats, flats_dev = [], []
    for q in range(P):
        bits = wide_bf16(rng, sum(numel))
        grads = [bits[s:s + k] for s, k in zip(pre, numel)]
        flats.append(opack.pack(oplan, grads))
        f = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, [dev(gq) for gq in grads], f)
        flats_dev.append(f)
    for r in sorted({0, P // 2, P - 1}):
        ref = reduce_mean([opack.owner_view(oplan, f, r) for f in flats], r)
        g, part = reduce(plan, r, flats_dev, G.LAYOUT_BUCKET_FLAT, S)
        assert_bits(g, ref, f"burst bucket-flat P={P} owner {r}")
        check_partial(part, ref, f"burst bucket-flat P={P} owner {r}")


@pytest.mark.parametrize("P", [24, 64, 100])
def test_burst_bf16_wire(P):
    rng = np.random.default_rng([47, P])
    plan = G.Plan([int(rng.integers(2 * CHUNK, 3 * CHUNK)) * P], 1 << 40, P, 8).upload()
    S = plan.shard_len
    r = P // 2
    cs = [wide_bf16(rng, S) for _ in range(P)]
    ref = reduce_mean_bf16_wire(cs, r)
    g, part = reduce(plan, r, [dev(c) for c in cs], G.LAYOUT_SHARD_COMPACT, S, wire=True)
    assert_bits(g, ref, f"burst bf16 wire P={P}")
    check_partial(part, ref, f"burst bf16 wire P={P}")
    gi, _ = reduce(plan, r, [dev(interleave(cs, P, S))], G.LAYOUT_RANK_INTERLEAVED, S, wire=True)
    assert_bits(gi, ref, f"burst bf16 wire interleaved P={P}")


@pytest.mark.parametrize("S", [8, 504, 512, 520, 4096, CHUNK - 8, CHUNK, CHUNK + 8, 2 * CHUNK])
def test_burst_small_and_exact_shards(S):
    """Shards below one chunk, one row, and exact multiples of the chunk."""
    P = 64
    rng = np.random.default_rng([53, S])
    plan = G.Plan([S * P], 1 << 40, P, 8).upload()
    assert plan.shard_len == S
    cs = [wide_bf16(rng, S) for _ in range(P)]
    for r in (0, 37):
        ref = reduce_mean(cs, r)
        g, part = reduce(plan, r, [dev(c) for c in cs], G.LAYOUT_SHARD_COMPACT, S)
        assert_bits(g, ref, f"burst S={S} owner {r}")
        check_partial(part, ref, f"burst S={S} owner {r}")


@pytest.mark.parametrize("limit", [1, 3, 7, 9, 20])
def test_burst_capped_grids(limit):
    """Fewer blocks than chunks: each block walks several chunks, and below 8
    blocks some XCD classes have none (their chunk shares are empty)."""
    P = 32
    rng = np.random.default_rng([59, limit])
    plan = G.Plan([int(11.5 * CHUNK) * P + 40], 1 << 40, P, 8).upload()
    S = plan.shard_len
    cs = [wide_bf16(rng, S) for _ in range(P)]
    r = 5
    ref = reduce_mean(cs, r)
    G.set_grid_limit(limit)
    g, part = reduce(plan, r, [dev(c) for c in cs], G.LAYOUT_SHARD_COMPACT, S)
    assert_bits(g, ref, f"burst, grid capped at {limit}")
    check_partial(part, ref, f"burst, grid capped at {limit}")
    gi, _ = reduce(plan, r, [dev(interleave(cs, P, S))], G.LAYOUT_RANK_INTERLEAVED, S)
    assert_bits(gi, ref, f"burst interleaved, grid capped at {limit}")


def test_burst_noalloc_entry_point():
    P = 64
    rng = np.random.default_rng(61)
    plan = G.Plan([int(2.3 * CHUNK) * P], 1 << 40, P, 8).upload()
    S = plan.shard_len
    cs = [wide_bf16(rng, S) for _ in range(P)]
    r = 63
    ref = reduce_mean(cs, r)
    src = [dev(c) for c in cs]
    try:
        for pw in WRITES:
            G.set_burst_window(*pw)
            g = torch.full((S,), float("nan"), dtype=torch.float32, device="cuda")
            part = torch.zeros(1, dtype=torch.float64, device="cuda")
            G.shard_reduce_mean_noalloc(plan, r, src, G.LAYOUT_SHARD_COMPACT, g, part)
            torch.cuda.synchronize()
            assert_bits(host(g), ref, f"burst, no-allocation entry point, writes {pw}")
            check_partial(float(host(part)[0]), ref, f"burst, no-allocation entry point, writes {pw}")
    finally:
        G.set_burst_window(0, 0)


@pytest.mark.parametrize("P", [24, 33])
def test_product_rule_at_its_threshold(P):
    """Without the forcing hook, a shard of exactly 2^23 elements takes the
    burst kernel (its norm partial has the burst grid's grouping, bit for bit)
    and 8 elements fewer take the tile kernel, at an unrolled P and at one on
    the runtime-P loop; g equals the oracle either way."""
    rng = np.random.default_rng([67, P])
    G.set_reduce_path(G.REDUCE_PATH_BY_SIZE)
    for S in (1 << 23, (1 << 23) - 8):
        plan = G.Plan([S * P], 1 << 40, P, 8).upload()
        assert plan.shard_len == S
        # bf16 bits with exponents 2^-27..2^12 and either sign: finite, quick to draw
        cs = [(rng.integers(100, 140, S, dtype=np.uint16) << 7 | rng.integers(0, 128, S, dtype=np.uint16)
               | (rng.integers(0, 2, S, dtype=np.uint16) << 15)).astype(np.uint16) for _ in range(P)]
        dev_cs = [dev(c) for c in cs]
        r = 11
        ref = reduce_mean(cs, r)
        g, part = reduce(plan, r, dev_cs, G.LAYOUT_SHARD_COMPACT, S)
        assert_bits(g, ref, f"product rule, S={S}")
        check_partial(part, ref, f"product rule, S={S}")
        G.set_reduce_path(G.REDUCE_PATH_BURST)
        _, part_burst = reduce(plan, r, dev_cs, G.LAYOUT_SHARD_COMPACT, S)
        G.set_reduce_path(G.REDUCE_PATH_TILE)
        _, part_tile = reduce(plan, r, dev_cs, G.LAYOUT_SHARD_COMPACT, S)
        G.set_reduce_path(G.REDUCE_PATH_BY_SIZE)
        want = part_burst if S >= 1 << 23 else part_tile
        assert part == want, (S, part, part_burst, part_tile)
        assert part_burst != part_tile or S < 4096, "the two groupings should differ in the last bits"
        del dev_cs


@pytest.mark.parametrize("seed", range(6))
def test_burst_random_plans(seed):
    """Random plans (1-40 tensors of 0-20,000 elements, caps 2-400 KB, align 8
    or 64) at the burst kernel's world sizes, bucket-flat contributions, three
    owners each, against the oracle."""
    rng = np.random.default_rng([71, seed])
    P = int(rng.choice([24, 32, 64, 96]))
    align = int(rng.choice([8, 64]))
    numel = [int(x) for x in rng.integers(0, 20000, int(rng.integers(1, 41)))]
    cap = int(rng.integers(2_000, 400_000))
    plan = G.Plan(numel, cap, P, align).upload()
    oplan = make_plan(numel, cap, P, align)
    S = plan.shard_len
    say(f"seed {seed}: P={P} align={align} tensors={len(numel)} buckets={plan.n_buckets} S={S}")
    pre = OI.prefix(numel)
    flats, flats_dev = [], []
    for q in range(P):
        bits = wide_bf16(rng, sum(numel))
        grads = [bits[s:s + k] for s, k in zip(pre, numel)]
        flats.append(opack.pack(oplan, grads))
        f = torch.full((plan.flat_len,), 0x7f7f, dtype=torch.int16, device="cuda").view(torch.uint16)
        G.bucket_pack(plan, [dev(gq) for gq in grads], f)
        flats_dev.append(f)
    for r in sorted({0, P - 1, int(rng.integers(0, P))}):
        ref = reduce_mean([opack.owner_view(oplan, f, r) for f in flats], r)
        g, part = reduce(plan, r, flats_dev, G.LAYOUT_BUCKET_FLAT, S)
        assert_bits(g, ref, f"burst, random plan {seed}, owner {r}")
        check_partial(part, ref, f"burst, random plan {seed}, owner {r}")
