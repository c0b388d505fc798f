"""Full-coverage GPU parity at the full sizes, in the launch configuration
bench.py times: the 1.3B model and the 7B share (P = 8, bucket-flat
contributions, bf16 parameters in all-gather layout) and the 70B share (P =
64, shard-compact contributions, shard-layout bf16): every owner of the 1.3B
model, owner 0 and the last owner of the 7B share (whose chunk of every bucket
ends where the bucket does and whose ring order starts at rank 0), owner 0 of
the 70B share.  (The pads of the padded workloads are checked on every owner
at the small sizes.)
Every shard element is compared with the oracle, window by window (16M elements): the
reduced gradient g, the updated master, m and v and the bf16 parameters bit
for bit; the fused fp64 norm partial against the oracle's partial of the
whole shard within 1e-5 relative.

The step is the one "Distributed Training: Data Parallel, Model Parallel and
FSDP Strategies" (Inside DDP) describes: the global norm is clipped, then AdamW
runs, so the oracle's AdamW takes the clip coefficient the GPU's k_clip formed
from the GPU's partials, and the oracle reproduces that coefficient from the
GPU's total bit for bit.  The other ranks' partials are stand-ins equal to
this shard's (the exchange is not simulated).

The oracle regenerates each window's inputs on the host from the seeded
generator (placed with the oracle's plan) and runs on one slice per host
thread; GPU inputs come from the device generator placed with the library's
plan.  The 70B share's rank-interleaved receive layout is checked against the
shard-compact g at the full size too.

The unsharded (DDP) step of the 1.3B model is held to the same bar on every
flat position, in the configuration bench.py --variant ddp times: the
all-reduce mean (each chunk summed in the ring order that ends at its owner),
the P chunk owners' fused norm partials against the oracle's, the clip from
those real partials, AdamW over the whole flat buffer and the unpacked bf16
parameters."""
import concurrent.futures as cf
import os
import time

import numpy as np
import pytest
import torch

import gradient_sync_zero_amd as G
from oracle.adamw import adamw
from oracle.norm import clip_coef as o_clip, sqnorm_partial
from oracle.plan import make_plan
from oracle.reduce import reduce_mean
from synth import gen
from synth import workloads as W
from tests import gpu_inputs as GI
from tests import oracle_inputs as OI
from tests.parity import assert_bits, host

pytestmark = pytest.mark.gpu

WINDOW = 1 << 24
THREADS = max(1, min(16, os.cpu_count() or 1))


def say(*a):
    print(*a, flush=True)


class GpuStep:
    """The GPU side of one workload's step, run once: device outputs kept for
    the window comparisons, the contributions freed."""

    def __init__(self, cfg, owner):
        w = W.by_id(cfg)
        P, r = w.world_size, owner
        plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
        S, L = plan.shard_len, plan.flat_len
        flat = (P + 2) * 2 * L + 2 * w.n_params + 18 * S < 240e9      # as bench.py decides
        t0 = time.perf_counter()
        if flat:
            gbuf = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
            flats = [torch.empty(L, dtype=torch.uint16, device="cuda") for _ in range(P)]
            for q in [q for q in range(P - 1, -1, -1) if q != r] + [r]:
                _, views = GI.rank_grads(w, q, gbuf)
                G.bucket_pack(plan, views, flats[q])
            del gbuf, views
            contribs, lay = flats, G.LAYOUT_BUCKET_FLAT
            gathered = torch.full((L,), 0x7777, dtype=torch.uint16, device="cuda")
            shard_out = None
        else:
            contribs, lay = GI.compact_contribs(plan, w, r), G.LAYOUT_SHARD_COMPACT
            gathered = None
            shard_out = torch.full((S,), 0x7777, dtype=torch.uint16, device="cuda")
        self.master, self.m, self.v = GI.owner_state(plan, w, r)
        self.g = torch.empty(S, dtype=torch.float32, device="cuda")
        ws = torch.zeros(G.workspace_bytes(S) // 8, dtype=torch.float64, device="cuda")
        partials = torch.zeros(P, dtype=torch.float64, device="cuda")
        G.shard_reduce_mean(plan, r, contribs, lay, self.g, partials[r:r + 1], ws)
        torch.cuda.synchronize()
        partials.fill_(float(partials[r]))                      # the other ranks' stand-ins
        coef = torch.empty(1, dtype=torch.float32, device="cuda")
        norm = torch.empty(1, dtype=torch.float32, device="cuda")
        tot = torch.empty(1, dtype=torch.float64, device="cuda")
        G.clip_coef(partials, w.hp.max_norm, coef, norm, tot)
        G.shard_adamw_step(plan, r, self.master, self.m, self.v, self.g, coef, w.hp, gathered,
                           shard_out)
        torch.cuda.synchronize()
        self.partial = float(host(partials)[r])
        self.coef, self.norm, self.total = host(coef)[0], host(norm)[0], float(host(tot)[0])
        self.ilv_same = None
        if not flat:
            # the same values in one rank-interleaved receive buffer: the same g
            # and partial bit for bit (after the compact buffers are freed)
            del contribs
            torch.cuda.empty_cache()
            ibuf = GI.interleaved_contribs(plan, w, r, G.interleaved_len(plan))
            g2 = torch.empty_like(self.g)
            p2 = torch.zeros(1, dtype=torch.float64, device="cuda")
            G.shard_reduce_mean(plan, r, [ibuf], G.LAYOUT_RANK_INTERLEAVED, g2, p2, ws)
            torch.cuda.synchronize()
            self.ilv_same = (bool(torch.equal(g2.view(torch.int32), self.g.view(torch.int32))),
                             float(host(p2)[0]) == self.partial)
            del ibuf, g2
        else:
            del contribs, flats
        torch.cuda.empty_cache()
        self.w, self.plan, self.S, self.flat, self.owner = w, plan, S, flat, r
        self.gathered, self.shard_out = gathered, shard_out
        say(f"[{w.name}] owner {r}: GPU step done in {time.perf_counter() - t0:.1f} s: S={S}, "
            f"partial={self.partial:.6e}, norm={self.norm}, coef={self.coef}")


class OracleWindows:
    """The oracle side: one owner's shard (or, with flat=True, the whole
    bucket-major flat buffer) in windows, regenerated on the host."""

    def __init__(self, w, flat=False, owner=0):
        self.w, self.owner = w, owner
        self.plan = make_plan(w.numel, w.bucket_cap_bytes, w.world_size)
        if flat:   # (flat offset, parameter index, length) of every tensor
            pre = OI.prefix(w.numel)
            self.pieces = sorted((self.plan.tensor_offset[t], pre[t], n)
                                 for t, n in enumerate(w.numel) if n)
        else:
            self.pieces = sorted(OI.owner_pieces(self.plan, owner))
        self.starts = np.array([p[0] for p in self.pieces], dtype=np.int64)
        self.pool = cf.ThreadPoolExecutor(max_workers=THREADS)

    def fill(self, a, b, kind, rank, std, mode):
        """Generator values of shard elements [a, b) (zero at pads)."""
        out = np.zeros(b - a, dtype=np.uint16 if mode == gen.MODE_BF16 else np.float32)
        k = max(int(np.searchsorted(self.starts, a, side="right")) - 1, 0)
        for so, pi, n in self.pieces[k:]:
            if so >= b:
                break
            lo, hi = max(so, a), min(so + n, b)
            if lo < hi:
                gen.host_fill(self.w.cfg_id, kind, rank, pi + (lo - so), hi - lo, std, mode,
                              out=out[lo - a:hi - a])
        return out

    def slices(self, n):
        per = -(-n // THREADS)
        step = (per + 7) // 8 * 8
        return [(s, min(s + step, n)) for s in range(0, n, step)]

    def window(self, a, b, coef):
        """g, partial, theta, m, v, bf16 of shard elements [a, b)."""
        w = self.w
        cs = [self.fill(a, b, W.KIND_GRAD, q, w.grad_std, gen.MODE_BF16)
              for q in range(w.world_size)]
        st = [self.fill(a, b, kind, 0, std, mode) for kind, std, mode in OI.STATE_KINDS]
        hp = w.hp

        def run(sl):
            lo, hi = sl
            g = reduce_mean([c[lo:hi] for c in cs], self.owner)
            th, m, v, p = adamw(st[0][lo:hi], st[1][lo:hi], st[2][lo:hi], g, coef, hp.lr,
                                hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step)
            return g, th, m, v, p

        parts = list(self.pool.map(run, self.slices(b - a)))
        out = [np.concatenate([p[k] for p in parts]) for k in range(5)]
        return out[0], sqnorm_partial(out[0]), out[1], out[2], out[3], out[4]


_cache = {}


def step_for(cfg, owner=0):
    if (cfg, owner) not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        _cache[cfg, owner] = (GpuStep(cfg, owner), OracleWindows(W.by_id(cfg), owner=owner), {})
    return _cache[cfg, owner]


def compare_windows(cfg, part, n_parts, owner=0):
    gs, ow, acc = step_for(cfg, owner)
    S = gs.S
    nwin = -(-S // WINDOW)
    lo_w, hi_w = part * nwin // n_parts, (part + 1) * nwin // n_parts
    t0 = time.perf_counter()
    for k in range(lo_w, hi_w):
        a, b = k * WINDOW, min((k + 1) * WINDOW, S)
        g, sq, th, m, v, p = ow.window(a, b, gs.coef)
        acc[k] = sq
        assert_bits(host(gs.g[a:b]), g, f"{gs.w.name} g [{a}, {b})")
        assert_bits(host(gs.master[a:b]), th, f"{gs.w.name} master [{a}, {b})")
        assert_bits(host(gs.m[a:b]), m, f"{gs.w.name} m [{a}, {b})")
        assert_bits(host(gs.v[a:b]), v, f"{gs.w.name} v [{a}, {b})")
        if gs.flat:
            pos = OI.flat_pos_of_shard(ow.plan, owner, np.arange(a, b, dtype=np.int64))
            idx = torch.from_numpy(pos).to("cuda")
            got = host(gs.gathered.view(torch.int16)[idx].view(torch.uint16))
        else:
            got = host(gs.shard_out[a:b])
        assert_bits(got, p, f"{gs.w.name} bf16 [{a}, {b})")
        if k % 8 == 0 or k == hi_w - 1:
            say(f"[{gs.w.name}] windows {lo_w}..{k} of {nwin} equal ({time.perf_counter() - t0:.1f} s)")


def check_norm_and_clip(cfg, owner=0):
    gs, ow, acc = step_for(cfg, owner)
    nwin = -(-gs.S // WINDOW)
    assert sorted(acc) == list(range(nwin)), "every window compared first"
    want = 0.0
    for k in range(nwin):                      # the shard's partial, window by window
        want = want + acc[k]
    assert abs(gs.partial - want) <= 1e-5 * want, (gs.partial, want)
    # the GPU's clip coefficient from the GPU's total, reproduced by the oracle
    assert o_clip(gs.total, gs.w.hp.max_norm) == (gs.norm, gs.coef)
    own = o_clip(want * gs.w.world_size, gs.w.hp.max_norm)
    say(f"[{gs.w.name}] partial {gs.partial!r} vs oracle {want!r} "
        f"(rel {abs(gs.partial - want) / want:.2e}); coef {gs.coef!r}, oracle's own {own[1]!r}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("owner", range(8))
def test_gpt_1_3b_every_shard_element(owner):
    assert W.by_id(2).world_size == 8
    compare_windows(2, 0, 1, owner)
    check_norm_and_clip(2, owner)
    if owner == 7:
        _cache.clear()
        torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("part", [0, 1])
def test_llama_7b_share_every_shard_element(part):
    compare_windows(3, part, 2)
    if part == 1:
        check_norm_and_clip(3)


@pytest.mark.timeout(900)
def test_llama_7b_share_last_owner_every_shard_element():
    last = W.by_id(3).world_size - 1
    compare_windows(3, 0, 1, last)
    check_norm_and_clip(3, last)
    _cache.clear()
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("part", [0, 1, 2, 3])
def test_llama_70b_share_every_shard_element(part):
    gs = step_for(4)[0]
    if part == 0:
        assert gs.ilv_same == (True, True), "interleaved receive layout differs from shard-compact"
    compare_windows(4, part, 4)
    if part == 3:
        check_norm_and_clip(4)
        _cache.clear()
        torch.cuda.empty_cache()


# ---------------------------------------------------------------- the DDP step

class GpuDdpStep:
    """The unsharded (DDP / NO_SHARD) step of bench.py --variant ddp, run once:
    pack, all-reduce mean with the P chunk owners' fused norm partials, clip
    from those partials, AdamW over the whole flat buffer, unpack."""

    def __init__(self, cfg):
        w = W.by_id(cfg)
        P = w.world_size
        plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
        L = plan.flat_len
        t0 = time.perf_counter()
        gbuf = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
        flats = [torch.empty(L, dtype=torch.uint16, device="cuda") for _ in range(P)]
        for q in range(P):
            _, views = GI.rank_grads(w, q, gbuf)
            G.bucket_pack(plan, views, flats[q])
        del gbuf, views
        self.master, self.m, self.v = GI.full_state(plan, w)
        self.g = torch.empty(L, dtype=torch.float32, device="cuda")
        ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")
        partials = torch.zeros(P, dtype=torch.float64, device="cuda")
        coef = torch.empty(1, dtype=torch.float32, device="cuda")
        norm = torch.empty(1, dtype=torch.float32, device="cuda")
        tot = torch.empty(1, dtype=torch.float64, device="cuda")
        pflat = torch.full((L,), 0x7777, dtype=torch.uint16, device="cuda")
        self.pbuf = torch.full((w.n_params,), 0x7777, dtype=torch.uint16, device="cuda")
        params = [self.pbuf[s0:s0 + n] for s0, n in zip(GI.prefix(w.numel), w.numel)]
        G.allreduce_mean(plan, flats, self.g, partials, ws)
        G.clip_coef(partials, w.hp.max_norm, coef, norm, tot)
        G.adamw_step(self.master, self.m, self.v, self.g, coef, w.hp, pflat)
        G.bucket_unpack(plan, pflat, params)
        torch.cuda.synchronize()
        self.partials = host(partials).astype(np.float64)
        self.coef, self.norm, self.total = host(coef)[0], host(norm)[0], float(host(tot)[0])
        del flats, pflat, params
        torch.cuda.empty_cache()
        self.w, self.L = w, L
        say(f"[{w.name} DDP] GPU step done in {time.perf_counter() - t0:.1f} s: L={L}, "
            f"total={self.total:.6e}, coef={self.coef}")


def ring_segments(oplan):
    """(flat start, end, chunk owner) of every chunk: the all-reduce sums chunk c
    of every bucket in the ring order that ends at rank c."""
    out = []
    for b, bk in enumerate(oplan.buckets):
        for c in range(oplan.world_size):
            cs, ce = oplan.chunk_range(b, c)
            if cs < ce:
                out.append((cs, ce, c))
    return out


_ddp = {}


def compare_ddp_windows(cfg, part, n_parts):
    if cfg not in _ddp:
        _ddp.clear()
        torch.cuda.empty_cache()
        ow = OracleWindows(W.by_id(cfg), flat=True)
        _ddp[cfg] = (GpuDdpStep(cfg), ow, ring_segments(ow.plan), {})
    gs, ow, segs, acc = _ddp[cfg]
    w, L, P = gs.w, gs.L, gs.w.world_size
    seg_starts = np.array([sg[0] for sg in segs], dtype=np.int64)
    pre = OI.prefix(w.numel)
    nwin = -(-L // WINDOW)
    lo_w, hi_w = part * nwin // n_parts, (part + 1) * nwin // n_parts
    hp = w.hp
    t0 = time.perf_counter()
    for k in range(lo_w, hi_w):
        a, b = k * WINDOW, min((k + 1) * WINDOW, L)
        cs = [ow.fill(a, b, W.KIND_GRAD, q, w.grad_std, gen.MODE_BF16) for q in range(P)]
        st = [ow.fill(a, b, kind, 0, std, mode) for kind, std, mode in OI.STATE_KINDS]
        # the window cut at chunk boundaries; each piece summed in its owner's ring order
        pieces = []
        j = max(int(np.searchsorted(seg_starts, a, side="right")) - 1, 0)
        for s0, e0, c in segs[j:]:
            if s0 >= b:
                break
            lo, hi = max(s0, a) - a, min(e0, b) - a
            for x in range(lo, hi, 1 << 20):          # slices of at most 1M for the threads
                pieces.append((x, min(x + (1 << 20), hi), c))

        def run(piece):
            lo, hi, c = piece
            g = reduce_mean([x[lo:hi] for x in cs], c)
            th, m, v, p = adamw(st[0][lo:hi], st[1][lo:hi], st[2][lo:hi], g, gs.coef, hp.lr,
                                hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step)
            return c, sqnorm_partial(g), g, th, m, v, p

        res = list(ow.pool.map(run, pieces))
        for c, sq, *_ in res:
            acc.setdefault(c, []).append((k, sq))
        out = [np.concatenate([r[i] for r in res]) for i in range(2, 7)]
        assert_bits(host(gs.g[a:b]), out[0], f"DDP g [{a}, {b})")
        assert_bits(host(gs.master[a:b]), out[1], f"DDP master [{a}, {b})")
        assert_bits(host(gs.m[a:b]), out[2], f"DDP m [{a}, {b})")
        assert_bits(host(gs.v[a:b]), out[3], f"DDP v [{a}, {b})")
        # the unpacked parameters: flat position f of tensor t is parameter pre_t + (f - off_t)
        pidx = OI.param_index_of_flat(ow.plan, np.arange(a, b, dtype=np.int64))
        real = pidx >= 0
        got = host(gs.pbuf.view(torch.int16)[torch.from_numpy(pidx[real]).to("cuda")]
                   .view(torch.uint16))
        assert_bits(got, out[4][real], f"DDP unpacked bf16 [{a}, {b})")
        assert not out[0][~real].any() and not out[1][~real].any()      # pads stay 0
        if k % 8 == 0 or k == hi_w - 1:
            say(f"[{w.name} DDP] windows {lo_w}..{k} of {nwin} equal ({time.perf_counter() - t0:.1f} s)")
    if part == n_parts - 1:
        # each chunk owner's fused partial against the oracle's, window order
        for c in range(P):
            want = 0.0
            for _, sq in sorted(acc[c]):
                want = want + sq
            assert abs(gs.partials[c] - want) <= 1e-5 * want, (c, gs.partials[c], want)
        assert o_clip(gs.total, w.hp.max_norm) == (gs.norm, gs.coef)
        say(f"[{w.name} DDP] {P} partials within {max(abs(gs.partials[c] - sum(s for _, s in acc[c])) / gs.partials[c] for c in range(P)):.1e}; coef {gs.coef!r}")
        _ddp.clear()
        torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("part", [0, 1])
def test_gpt_1_3b_ddp_step_every_flat_position(part):
    compare_ddp_windows(2, part, 2)
