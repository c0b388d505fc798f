"""The allocation-free shard reduce, gsz_shard_reduce_mean_noalloc (for
callers that cannot allocate device memory), against the workspace form
gsz_shard_reduce_mean through the C ABI: the same reduced gradient and fp64
norm partial bit for bit, on calls in a row with a smaller shard after a
larger one (the fixed scratch keeps the previous call's partials), for both
reduce kernels (P <= 16 and P = 64) and both contribution layouts; a shard
over the variant's limit is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import gradient_sync_zero_amd as G
from synth import workloads as W
from tests import gpu_inputs as GI
from tests.parity import assert_bits, host

pytestmark = pytest.mark.gpu


def flat_contribs(plan, w):
    flats = []
    gbuf = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
    for q in range(w.world_size):
        _, views = GI.rank_grads(w, q, gbuf)
        f = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, views, f)
        flats.append(f)
    return flats


def both_forms(plan, r, contribs, layout):
    """(g, partial) from the workspace form, then from the allocation-free form."""
    S = plan.shard_len
    ws = torch.full((G.workspace_bytes(S) // 8,), float("nan"), dtype=torch.float64, device="cuda")
    out = []
    for noalloc in (False, True):
        g = torch.full((S,), float("nan"), dtype=torch.float32, device="cuda")
        part = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
        if noalloc:
            G.shard_reduce_mean_noalloc(plan, r, contribs, layout, g, part)
        else:
            G.shard_reduce_mean(plan, r, contribs, layout, g, part, ws)
        torch.cuda.synchronize()
        out.append((host(g), host(part)[0]))
    return out


def check(plan, r, contribs, layout, what):
    (g0, p0), (g1, p1) = both_forms(plan, r, contribs, layout)
    assert_bits(g1, g0, f"{what}: g")
    assert p1 == p0 and np.isfinite(p1) and p1 > 0, (what, p0, p1)
    print(f"{what}: S={plan.shard_len}, partial {p1!r}: equal", flush=True)


def test_noalloc_equals_workspace_form_on_consecutive_calls():
    # a larger shard first (GPT-2 small, P = 8, bucket-flat), then smaller ones
    w = W.by_id(1)
    plan = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size).upload()
    flats = flat_contribs(plan, w)
    check(plan, 3, flats, G.LAYOUT_BUCKET_FLAT, "gpt2-small P=8 owner 3, bucket-flat")
    t = W.tiny()
    tplan = G.Plan(t.numel, t.bucket_cap_bytes, t.world_size).upload()
    check(tplan, 1, GI.compact_contribs(tplan, t, 1), G.LAYOUT_SHARD_COMPACT,
          "tiny P=4 owner 1, shard-compact")
    # the 16-byte-load kernel (P = 64), smaller again
    rng = np.random.default_rng(5)
    plan64 = G.Plan([100_000], 1 << 40, 64, 8).upload()
    cs = [torch.from_numpy(rng.integers(0x3000, 0x3c00, plan64.shard_len, dtype=np.int32)
                           .astype(np.int16)).to("cuda").view(torch.uint16) for _ in range(64)]
    check(plan64, 63, cs, G.LAYOUT_SHARD_COMPACT, "P=64 owner 63, shard-compact")
    # and the larger shard again after the small ones
    check(plan, 0, flats, G.LAYOUT_BUCKET_FLAT, "gpt2-small P=8 owner 0, bucket-flat")


def test_noalloc_refuses_a_shard_over_its_limit():
    big = G.Plan([(1 << 31) + 64], 1 << 40, 1)     # S = 2^31 + 64: host plan only
    assert big.shard_len > 1 << 31
    lib = G.load()
    arr = (ctypes.c_void_p * 1)(None)
    assert lib.gsz_shard_reduce_mean_noalloc(big.handle, 0, arr, G.LAYOUT_SHARD_COMPACT, None,
                                             None, None) == -3          # GSZ_ERR_SIZE
    assert b"limit" in lib.gsz_last_error()
