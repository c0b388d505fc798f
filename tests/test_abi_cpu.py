"""CPU tests of the C ABI: the library loads and exports every symbol the
header declares; the C++ planner reproduces the oracle's plan exactly; the
plan hash detects ranks that disagree (failure injection: a rank that skips an
unused parameter); ledger and argument validation.  No device call is made."""
import ctypes
import os
import re

import numpy as np
import pytest

import gradient_sync_zero_amd as G
from oracle import ledger as oledger
from oracle.plan import make_plan
from synth import workloads as W

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
HEADER = os.path.join(INCLUDE, "gsz.h")
TEST_HEADER = os.path.join(INCLUDE, "gsz_test.h")
CSRC = os.path.join(os.path.dirname(G.LIB_PATH), "csrc")


def declared_symbols(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(gsz_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert len(syms) >= 17
    lib = ctypes.CDLL(G.LIB_PATH)
    missing = [s for s in syms if not hasattr(lib, s)]
    assert not missing, missing
    for s in ("gsz_bucket_pack", "gsz_shard_reduce_mean", "gsz_shard_grad_sqnorm",
              "gsz_clip_coef", "gsz_shard_adamw_step", "gsz_allgather_layout_write",
              "gsz_plan_device_bytes", "gsz_plan_upload"):
        assert s in syms


def test_test_hooks_live_only_in_the_test_build():
    """The grid cap is process-wide state, so the product library does not
    have it; the test build exports everything the product does plus the
    hooks of gsz_test.h."""
    hooks = declared_symbols(TEST_HEADER)
    assert hooks == ["gsz_test_max_tile_span", "gsz_test_set_burst_window",
                     "gsz_test_set_flat_wide", "gsz_test_set_grid_limit",
                     "gsz_test_set_reduce_path"]
    prod = ctypes.CDLL(G.LIB_PATH)
    test = ctypes.CDLL(G._binding.TEST_LIB_PATH)
    assert not any(hasattr(prod, h) for h in hooks)
    assert all(hasattr(test, s) for s in declared_symbols() + hooks)
    with pytest.raises(RuntimeError):
        G.set_grid_limit(4)                      # outside test_hooks(): refused
    with pytest.raises(RuntimeError):
        G.set_reduce_path(G.REDUCE_PATH_BURST)
    with pytest.raises(RuntimeError):
        G.set_burst_window(64, 8)
    with pytest.raises(RuntimeError):
        G.set_flat_wide(True)
    with G.test_hooks():
        G.set_flat_wide(True)
        G.set_flat_wide(False)
        with pytest.raises(G.GszError) as e:     # the cap is a count of blocks
            G.set_grid_limit(-1)
        assert "-1" in str(e.value)
        G.set_grid_limit(0)
        for bad in (-1, 3):
            with pytest.raises(G.GszError) as e:
                G.set_reduce_path(bad)
            assert str(bad) in str(e.value)
        G.set_reduce_path(G.REDUCE_PATH_BY_SIZE)
        for bad in (3, 100, (1 << 31) + 1):      # the period is a power of two (or 0)
            with pytest.raises(G.GszError) as e:
                G.set_burst_window(bad, 1)
            assert str(bad) in str(e.value)
        for good in ((0, 0), (1, 1), (64, 24), (1 << 31, 0)):
            G.set_burst_window(*good)
        G.set_burst_window(0, 0)
        p = G.Plan([5], 100, 2)
    with pytest.raises(ValueError):              # a plan is tied to its build
        G._binding._lib_for(p)


def _spans_brute_force(oplan, r, tile):
    """Largest flat span of `tile` consecutive shard elements of owner r, from
    the oracle's plan: each shard index's flat position, tile by tile."""
    offs = np.array([b.shard_off for b in oplan.buckets], dtype=np.int64)
    bases = np.array([b.base + r * b.chunk for b in oplan.buckets], dtype=np.int64)
    S = oplan.shard_len

    def pos(i):
        b = np.searchsorted(offs, i, side="right") - 1
        return bases[b] + (i - offs[b])

    first = np.arange(0, S, tile, dtype=np.int64)
    last = np.minimum(first + tile, S) - 1
    return int((pos(last) - pos(first) + 1).max())


@pytest.mark.parametrize("case", range(6))
def test_max_tile_span_matches_brute_force(case):
    """The span the library checks against 32-bit buffer offsets (its reduce
    and AdamW read and write bucket-flat buffers through descriptors based at
    each tile's first position) equals a brute-force count over every tile,
    for every owner and several tile sizes, including plans whose tiles cross
    several small buckets and one bucket holding a single large tensor."""
    rng = np.random.default_rng(900 + case)
    P = int(rng.choice([2, 3, 4, 8, 16]))
    T = int(rng.integers(3, 40))
    numel = [int(x) for x in rng.choice([0, 1, 7, 64, 500, 3000, 40000], size=T)]
    numel[int(rng.integers(T))] = int(rng.integers(1, 4)) * 1_000_003
    cap = int(rng.choice([256, 4096, 100_000, 25 << 20]))
    oplan = make_plan(numel, cap, P)
    if oplan.shard_len == 0:
        pytest.skip("empty shard")
    with G.test_hooks():
        plan = G.Plan(numel, cap, P)
        for r in range(P):
            for tile in (1, 64, 256, 2048, 5000):
                got = G.max_tile_span(plan, r, tile)
                assert got == _spans_brute_force(oplan, r, tile), (r, tile)
        with pytest.raises(G.GszError):
            G.max_tile_span(plan, P, 256)
        with pytest.raises(G.GszError):
            G.max_tile_span(plan, 0, 0)


def test_max_tile_span_reaches_the_32_bit_limit_on_a_huge_bucket():
    """A plan whose first bucket holds a tensor of 3 * 2^30 elements has, for
    owner 0 of 2, a 2048-element tile that crosses from that bucket's chunk to
    the next bucket's: it spans more than 2^30 flat positions (2^31 bytes of
    bf16), the case in which the product reads bucket-flat contributions and
    writes all-gather positions through 64-bit addresses.  Owner 1's chunks
    follow each other closely, and the 7B share stays far below the limit.
    Host only: the plan is metadata."""
    numel = [1000, 3 << 30, 1000]
    oplan = make_plan(numel, 25 << 20, 2)
    with G.test_hooks():
        plan = G.Plan(numel, 25 << 20, 2)
        spans = [G.max_tile_span(plan, r, 2048) for r in range(2)]
        assert spans == [_spans_brute_force(oplan, r, 2048) for r in range(2)]
        assert spans[0] * 2 >= 1 << 31 > spans[1] * 2, spans
        w = W.by_id(3)
        p7 = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size)
        assert G.max_tile_span(p7, 0, 2048) * 2 < 1 << 31


def test_library_neither_allocates_device_memory_nor_waits():
    """The library's sources make no device allocation, free or synchronising
    call: device memory is the caller's (plan tables, workspace), and every
    device call only enqueues work on the caller's stream."""
    banned = re.compile(r"\b(hipMalloc\w*|hipFree\w*|hipExtMalloc\w*|hipMallocManaged|"
                        r"hipHostMalloc|hipDeviceSynchronize|hipStreamSynchronize|"
                        r"hipEventSynchronize|hipMemcpy|hipMemset)\s*\(")
    for name in sorted(os.listdir(CSRC)):
        text = open(os.path.join(CSRC, name)).read()
        assert not banned.search(text), (name, banned.search(text).group(0))
    undefined = {line.split()[-1].split("@")[0] for line in
                 os.popen(f"nm -D --undefined-only {G.LIB_PATH}").read().splitlines() if line.strip()}
    assert "hipMemcpyAsync" in undefined and "hipLaunchKernel" in " ".join(undefined)
    assert not undefined & {"hipMalloc", "hipMallocAsync", "hipMallocManaged", "hipExtMallocWithFlags",
                            "hipHostMalloc", "hipFree", "hipFreeAsync", "hipHostFree", "hipMemcpy",
                            "hipMemset", "hipDeviceSynchronize", "hipStreamSynchronize",
                            "hipEventSynchronize"}


def test_noalloc_reduce_refuses_shards_over_its_fixed_scratch():
    """The allocation-free reduce has a fixed scratch for shards of at most
    2^31 elements; a larger plan is refused before any device call."""
    big = G.Plan([(1 << 31) + 64], 1 << 40, 1)
    assert big.shard_len > 1 << 31
    lib = G.load()
    arr = (ctypes.c_void_p * 1)(None)
    assert lib.gsz_shard_reduce_mean_noalloc(big.handle, 0, arr, G.LAYOUT_SHARD_COMPACT, None,
                                             None, None) == -3          # GSZ_ERR_SIZE
    assert b"2147483648" in lib.gsz_last_error()


def test_plan_device_bytes_is_the_documented_bound():
    """Header: at most 1,048,640 + 24 * n_tensors + 40 * n_buckets bytes."""
    for cfg in range(5):
        w = W.by_id(cfg)
        p = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size)
        nb = p.device_bytes()
        assert nb % 8 == 0 and nb <= 1048640 + 24 * p.n_tensors + 40 * p.n_buckets, cfg
    assert G.Plan([], 100, 2).device_bytes() > 0


def assert_same_plan(cplan, oplan):
    assert (cplan.flat_len, cplan.shard_len, cplan.n_buckets) == \
        (oplan.flat_len, oplan.shard_len, len(oplan.buckets))
    for b, ob in enumerate(oplan.buckets):
        cb = cplan.bucket(b)
        tensors = tuple(cb["first_tensor"] - k for k in range(cb["n_tensors"]))
        assert tensors == ob.tensors
        assert (cb["base"], cb["n_elems"], cb["padded"], cb["chunk"], cb["shard_off"]) == \
            (ob.base, ob.n, ob.padded, ob.chunk, ob.shard_off)
    for t in range(len(oplan.numel)):
        assert cplan.tensor(t) == (oplan.tensor_offset[t], oplan.tensor_bucket[t])


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_planner_matches_oracle_on_workloads(cfg):
    w = W.by_id(cfg)
    c = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size)
    o = make_plan(w.numel, w.bucket_cap_bytes, w.world_size)
    assert_same_plan(c, o)
    assert c.n_params == w.n_params


def test_planner_matches_oracle_on_random_cases():
    rng = np.random.default_rng(21)
    for _ in range(200):
        T = int(rng.integers(0, 40))
        numel = [int(x) for x in rng.integers(0, 5000, T)]
        if T and rng.random() < 0.3:
            numel[int(rng.integers(0, T))] = 0
        cap = int(rng.integers(1, 20000))
        P = int(rng.integers(1, 9))
        align = int(rng.choice([1, 2, 8, 64]))
        assert_same_plan(G.Plan(numel, cap, P, align), make_plan(numel, cap, P, align))


def fnv1a64(values):
    h = 0xcbf29ce484222325
    for x in values:
        for byte in int(x).to_bytes(8, "little", signed=True):
            h ^= byte
            h = (h * 0x100000001b3) & 0xFFFFFFFFFFFFFFFF
    return h


def test_plan_hash_is_fnv1a_of_the_canonical_description():
    w = W.tiny()
    c = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size)
    vals = [w.world_size, 64, w.bucket_cap_bytes, len(w.numel), *w.numel, c.n_buckets]
    for b in c.buckets():
        vals += [b["first_tensor"], b["n_tensors"], b["base"], b["n_elems"], b["padded"]]
    assert c.hash == fnv1a64(vals)
    assert fnv1a64([]) == 0xcbf29ce484222325


def test_plan_mismatch_is_an_error_not_a_hang():
    w = W.gpt2_small()
    ranks = [G.Plan(w.numel, w.bucket_cap_bytes, w.world_size) for _ in range(3)]
    for r in ranks[1:]:
        ranks[0].check(r.hash)                               # identical plans agree
    # one rank drops a parameter that took no part in its forward pass
    skipped = list(w.numel)
    skipped[5] = 0
    odd = G.Plan(skipped, w.bucket_cap_bytes, w.world_size)
    with pytest.raises(G.GszError) as e:
        ranks[0].check(odd.hash)
    assert e.value.name == "GSZ_ERR_PLAN_MISMATCH"
    for variant in (dict(cap=w.bucket_cap_bytes * 2), dict(P=4), dict(align=128)):
        p = G.Plan(w.numel, variant.get("cap", w.bucket_cap_bytes), variant.get("P", 8),
                   variant.get("align", 64))
        with pytest.raises(G.GszError):
            ranks[0].check(p.hash)


def test_ledger_matches_oracle():
    for P in (1, 2, 8, 64):
        for st in range(4):
            assert G.ledger_bytes_per_param(P, st) == oledger.bytes_per_param(P, st)
    with pytest.raises(G.GszError):
        G.ledger_bytes_per_param(0, 1)
    with pytest.raises(G.GszError):
        G.ledger_bytes_per_param(8, 4)


def test_argument_validation():
    with pytest.raises(G.GszError) as e:
        G.Plan([1, 2], 100, 0)
    assert e.value.name == "GSZ_ERR_INVALID_ARG"
    with pytest.raises(G.GszError):
        G.Plan([1, -2], 100, 2)
    with pytest.raises(G.GszError):
        G.Plan([1], 100, G.MAX_RANKS + 1)
    # sizes that would overflow the planner's int64 offsets are refused
    for sizes in ([1 << 48, 1], [(1 << 62), (1 << 62)], [(1 << 63) - 1]):
        with pytest.raises(G.GszError) as e:
            G.Plan(sizes, 100, 2)
        assert e.value.name == "GSZ_ERR_SIZE"
    big = G.Plan([1 << 47, 1 << 47], 1 << 40, 8)          # at the limit: a valid plan
    assert big.n_params == 1 << 48 and big.flat_len == 1 << 48
    p = G.Plan([5], 100, 2)
    with pytest.raises(G.GszError):
        p.bucket(1)
    with pytest.raises(G.GszError):
        p.tensor(-1)
    # one fp64 partial per 2048 elements (at most 2^23 of them, at least one)
    # plus 1024 second-stage sums
    for n, blocks in ((0, 1), (1, 1), (2048, 1), (2049, 2), (842301952, 411281),
                      (1077760128, 526251), (1 << 34, 1 << 23), ((1 << 34) + 1, 1 << 23)):
        assert G.workspace_bytes(n) == 8 * (blocks + 1024), n
    with pytest.raises(G.GszError):
        G.workspace_bytes(-1)
    lib = G.load()
    assert lib.gsz_status_string(-5) == b"plan mismatch"
    assert lib.gsz_plan_destroy(None) == 0


def test_binding_refuses_host_tensors():
    """The product path has no CPU fallback: host tensors are rejected before
    any call reaches the library."""
    import torch
    w = W.tiny()
    p = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size)
    grads = [torch.zeros(n, dtype=torch.bfloat16) for n in w.numel]
    with pytest.raises(ValueError):
        G.bucket_pack(p, grads, torch.zeros(p.flat_len, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        G.shard_reduce_mean(p, 0, [torch.zeros(p.shard_len, dtype=torch.bfloat16)] * 4,
                            G.LAYOUT_SHARD_COMPACT, torch.zeros(p.shard_len))
    with pytest.raises(ValueError):
        G.bucket_pack_f32(p, grads, torch.zeros(p.flat_len))
    with pytest.raises(ValueError):
        G.bucket_accumulate_f32(p, grads, torch.zeros(p.flat_len))
    with pytest.raises(ValueError):
        G.shard_reduce_mean_f32(p, 0, [torch.zeros(p.shard_len)] * 4, G.LAYOUT_SHARD_COMPACT,
                                torch.zeros(p.shard_len))


def test_torch_hip_runtime_is_loaded_before_the_library():
    """Loading the library in a fresh process must leave one HIP runtime
    mapped: torch's (the binding imports torch before loading libgsz)."""
    import subprocess
    import sys
    code = ("import gradient_sync_zero_amd, synth.gen as g; g._load_dev(); "
            "maps = open('/proc/self/maps').read(); "
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1"


def test_traffic_digest_covers_every_kernel_source():
    """The counter summaries are keyed to the kernel sources; a new header or
    HIP file under csrc/ must be part of that key."""
    import bench
    csrc = os.path.join(os.path.dirname(G.LIB_PATH), "csrc")
    on_disk = sorted(f for f in os.listdir(csrc) if f.endswith((".h", ".hip")))
    assert sorted(bench.KERNEL_SOURCES) == on_disk
    assert len(bench.kernel_source_digest()) == 64


def test_traffic_digest_ignores_comments_but_not_code():
    """A comment-only edit keeps a counter summary valid; any code edit, also
    inside a string literal, voids it."""
    import bench
    src = 'int f(int a) { // add one\n  return a + 1; /* done */ }\nconst char* s = "a // b";\n'
    same = 'int f(int a)   {\n  return a + 1;\n}\n// moved\nconst char* s = "a // b";'
    assert bench._code_tokens(src) == bench._code_tokens(same)
    for edited in (src.replace("a + 1", "a + 2"), src.replace('"a // b"', '"a // c"'),
                   src.replace("return", "return -")):
        assert bench._code_tokens(edited) != bench._code_tokens(src)


def test_planner_and_error_text_are_thread_safe():
    """Eight threads create plans concurrently (each checked against the
    oracle's planner) and provoke their own errors: the last-error text is per
    thread, so each sees its own message."""
    import threading
    failures = []

    def worker(k):
        rng = np.random.default_rng(100 + k)
        try:
            for i in range(40):
                T = int(rng.integers(1, 30))
                numel = [int(x) for x in rng.integers(0, 5000, T)]
                cap, P = int(rng.integers(1, 20000)), int(rng.integers(1, 9))
                assert_same_plan(G.Plan(numel, cap, P, 8), make_plan(numel, cap, P, 8))
                try:
                    G.Plan([1], 100, G.MAX_RANKS + 1 + k)            # a bad world size of its own
                except G.GszError:
                    msg = G.load().gsz_last_error().decode()
                    if str(G.MAX_RANKS + 1 + k) not in msg:
                        failures.append((k, i, msg))
        except Exception as e:                                        # noqa: BLE001
            failures.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not failures, failures[:3]


class _DevStandIn:
    """Stands in for a device tensor in the binding's host-side checks: it
    reports a dtype, a length and a device, and has no storage (address 0).  A
    call whose checks all pass reaches the library with NULL pointers, which it
    rejects before touching a device."""
    is_cuda = True

    def __init__(self, n, dtype):
        self._n, self.dtype = n, dtype

    def numel(self):
        return self._n

    def element_size(self):
        return 8 if "64" in str(self.dtype) else 4 if "32" in str(self.dtype) else 2

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return 0


def test_binding_checks_buffer_sizes_against_the_plan():
    """The library takes bare device pointers and cannot see buffer lengths; the
    binding checks every length the plan implies before the call, so a short
    (or, for per-tensor gradients, mis-sized) buffer is refused on the host
    instead of being read or written past its end on the GPU."""
    import torch
    w = W.tiny()
    p = G.Plan(w.numel, w.bucket_cap_bytes, w.world_size)
    S, L, P = p.shard_len, p.flat_len, p.world_size
    bf, f64 = torch.bfloat16, torch.float64
    D = _DevStandIn
    f = lambda n: D(n, torch.float32)
    b = lambda n: D(n, bf)
    grads = [b(n) for n in w.numel]
    short = list(grads)
    short[3] = b(w.numel[3] - 1)
    long_ = list(grads)
    long_[5] = b(w.numel[5] + 8)

    # stream=0 (the null stream) keeps torch's device runtime out of the calls
    def refused(fn, *args, match="elements"):
        with pytest.raises(ValueError, match=match):
            fn(*args, stream=0)

    def reaches_library(fn, *args):
        with pytest.raises(G.GszError):              # NULL pointers: refused by the library
            fn(*args, stream=0)

    unpack = lambda plan, params, flat, stream: G.bucket_unpack(plan, flat, params, stream=stream)
    for fn in (G.bucket_pack, G.bucket_accumulate, unpack):
        refused(fn, p, short, b(L))
        refused(fn, p, long_, b(L))
        refused(fn, p, grads, b(L - 1))
        refused(fn, p, grads[:-1], b(L), match="per plan tensor")
        reaches_library(fn, p, grads, b(L))
    for fn in (G.bucket_pack_f32, G.bucket_accumulate_f32):
        refused(fn, p, grads, f(L - 1))
        refused(fn, p, short, f(L))
        reaches_library(fn, p, grads, f(L))
    for layout, clen in ((G.LAYOUT_BUCKET_FLAT, L), (G.LAYOUT_SHARD_COMPACT, S)):
        cs = [b(clen)] * P
        cs_short = [b(clen)] * (P - 1) + [b(clen - 1)]
        refused(G.shard_reduce_mean, p, 0, cs_short, layout, f(S))
        refused(G.shard_reduce_mean, p, 0, cs, layout, f(S - 1))
        refused(G.shard_reduce_mean, p, 0, cs, layout, f(S), D(0, f64))
        reaches_library(G.shard_reduce_mean, p, 0, cs, layout, f(S))
        refused(G.shard_reduce_mean_f32, p, 0, [f(clen)] * (P - 1) + [f(clen - 1)], layout, f(S))
        refused(G.shard_reduce_mean_f32, p, 0, [f(clen)] * P, layout, f(S - 1))
        reaches_library(G.shard_reduce_mean_f32, p, 0, [f(clen)] * P, layout, f(S))
    refused(G.allreduce_mean, p, [b(L)] * (P - 1) + [b(L - 1)], f(L))
    refused(G.allreduce_mean, p, [b(L)] * P, f(L - 1))
    refused(G.allreduce_mean, p, [b(L)] * P, f(L), D(P - 1, f64))
    reaches_library(G.allreduce_mean, p, [b(L)] * P, f(L))
    refused(G.shard_grad_sqnorm, f(10), D(1, f64), D(1024, f64), 11)
    refused(G.shard_grad_sqnorm, f(10), D(0, f64), D(1024, f64))
    refused(G.clip_coef, D(P, f64), 1.0, f(0))
    coef = f(1)
    for k in range(4):                                # master, m, v, g
        st = [f(S) for _ in range(4)]
        st[k] = f(S - 1)
        refused(G.shard_adamw_step, p, 0, *st, coef, w.hp, b(L))
    refused(G.shard_adamw_step, p, 0, f(S), f(S), f(S), f(S), f(0), w.hp, b(L))
    refused(G.shard_adamw_step, p, 0, f(S), f(S), f(S), f(S), coef, w.hp, b(L - 1))
    refused(G.shard_adamw_step, p, 0, f(S), f(S), f(S), f(S), coef, w.hp, None, b(S - 1))
    reaches_library(G.shard_adamw_step, p, 0, f(S), f(S), f(S), f(S), coef, w.hp, b(L))
    refused(G.adamw_step, f(64), f(64), f(63), f(64), coef, w.hp, b(64))
    refused(G.adamw_step, f(64), f(64), f(64), f(64), coef, w.hp, b(56))
    reaches_library(G.adamw_step, f(64), f(64), f(64), f(64), coef, w.hp, b(64))
    refused(G.allgather_layout_write, p, 0, b(S - 1), b(L))
    refused(G.allgather_layout_write, p, 0, b(S), b(L - 1))
    reaches_library(G.allgather_layout_write, p, 0, b(S), b(L))
    # real host tensors of the right sizes are refused for being on the host
    grads_host = [torch.zeros(n, dtype=bf) for n in w.numel]
    refused(G.bucket_pack, p, grads_host, torch.zeros(L, dtype=bf), match="device tensor")


def test_binding_fails_loudly_without_the_library(tmp_path):
    """With libgsz.so absent the package refuses to import: there is no CPU
    fallback.  A copy of the package without the library is imported in a
    fresh process."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "gradient_sync_zero_amd"
    pkg.mkdir()
    src = os.path.dirname(G.LIB_PATH)
    for name in ("__init__.py", "_binding.py"):
        shutil.copy(os.path.join(src, name), pkg / name)
    code = ("try:\n"
            "    import gradient_sync_zero_amd as G\n"
            "except ImportError as e:\n"
            "    print('refused:', e)\n"
            "else:\n"
            "    print('ran without the library')\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=str(tmp_path), capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.startswith("refused:") and "no fallback" in out.stdout, out.stdout
