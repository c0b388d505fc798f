"""The shard step captured into a HIP graph (torch.cuda.graph) gives, replay
after replay, the bits of the same steps run eagerly: the library allocates
nothing, syncs nothing and records no memset inside a step.  Each replay is
followed by eager work and a synchronisation, and checked."""
import pytest
import torch

import gradient_sync_zero_amd as G
from synth import workloads as W
from tests import gpu_inputs as GI
from tests.parity import assert_bits, host

pytestmark = pytest.mark.gpu


def make_state(w, plan, owners):
    flats = []
    for q in range(w.world_size):
        f = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
        G.bucket_pack(plan, GI.rank_grads_separate(w, q), f)
        flats.append(f)
    states = {r: GI.owner_state(plan, w, r) for r in owners}
    return flats, states


@pytest.mark.parametrize("cfg,owners", [(0, (0, 1, 2, 3)), (1, (0,))])
def test_graph_replays_equal_eager_steps(cfg, owners):
    w = W.by_id(cfg)
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    my_grads = GI.rank_grads_separate(w, 0)
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")

    def buffers():
        flats, states = make_state(w, plan, owners)
        return dict(flats=flats, states=states,
                    g={r: torch.empty(plan.shard_len, device="cuda") for r in owners},
                    partials=torch.full((P,), 0.5, dtype=torch.float64, device="cuda"),
                    coef=torch.empty(1, device="cuda"),
                    gathered=torch.zeros(plan.flat_len, dtype=torch.uint16, device="cuda"))

    def step(b):
        G.bucket_pack(plan, my_grads, b["flats"][0])
        for r in owners:
            G.shard_reduce_mean(plan, r, b["flats"], G.LAYOUT_BUCKET_FLAT, b["g"][r],
                                b["partials"][r:r + 1], ws)
        G.clip_coef(b["partials"], w.hp.max_norm, b["coef"])
        for r in owners:
            th, m, v = b["states"][r]
            G.shard_adamw_step(plan, r, th, m, v, b["g"][r], b["coef"], w.hp, b["gathered"], None)

    def snapshot(b):
        torch.cuda.synchronize()
        out = [host(b["gathered"]), host(b["coef"])]
        for r in owners:
            out += [host(x) for x in b["states"][r]] + [host(b["g"][r])]
        return out

    eager = buffers()
    want = []
    for _ in range(3):
        step(eager)
        want.append(snapshot(eager))

    b = buffers()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(b)
    torch.cuda.synchronize()
    # capture recorded the work without running it: the state is still the initial one
    for k in range(3):
        graph.replay()
        junk = torch.randn(1 << 20, device="cuda").sum()        # eager work between replays
        torch.cuda.synchronize()
        got = snapshot(b)
        for i, (x, y) in enumerate(zip(got, want[k])):
            assert_bits(x, y, f"replay {k}, buffer {i}")
        del junk


@pytest.mark.parametrize("cfg", [0, 1])
def test_graph_replays_equal_eager_ddp_steps(cfg):
    """The unsharded step (pack, all-reduce with fused norm partials, clip,
    replicated AdamW, unpack) captured once and replayed."""
    w = W.by_id(cfg)
    P = w.world_size
    plan = G.Plan(w.numel, w.bucket_cap_bytes, P).upload()
    my_grads = GI.rank_grads_separate(w, 0)
    ws = torch.zeros(G.workspace_bytes(plan.shard_len) // 8, dtype=torch.float64, device="cuda")

    def buffers():
        flats = []
        for q in range(P):
            f = torch.empty(plan.flat_len, dtype=torch.uint16, device="cuda")
            G.bucket_pack(plan, GI.rank_grads_separate(w, q), f)
            flats.append(f)
        th, m, v = GI.full_state(plan, w)
        return dict(flats=flats, th=th, m=m, v=v,
                    g=torch.empty(plan.flat_len, device="cuda"),
                    parts=torch.full((P,), 0.5, dtype=torch.float64, device="cuda"),
                    coef=torch.empty(1, device="cuda"),
                    pflat=torch.zeros(plan.flat_len, dtype=torch.uint16, device="cuda"),
                    params=[torch.zeros(n, dtype=torch.uint16, device="cuda") for n in w.numel])

    def step(b):
        G.bucket_pack(plan, my_grads, b["flats"][0])
        G.allreduce_mean(plan, b["flats"], b["g"], b["parts"], ws)
        G.clip_coef(b["parts"], w.hp.max_norm, b["coef"])
        G.adamw_step(b["th"], b["m"], b["v"], b["g"], b["coef"], w.hp, b["pflat"])
        G.bucket_unpack(plan, b["pflat"], b["params"])

    def snapshot(b):
        torch.cuda.synchronize()
        return [host(b[k]) for k in ("g", "parts", "coef", "th", "m", "v", "pflat")] + \
               [host(t) for t in b["params"]]

    eager = buffers()
    want = []
    for _ in range(3):
        step(eager)
        want.append(snapshot(eager))

    b = buffers()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(b)
    torch.cuda.synchronize()
    for k in range(3):
        graph.replay()
        junk = torch.randn(1 << 20, device="cuda").sum()        # eager work between replays
        torch.cuda.synchronize()
        got = snapshot(b)
        for i, (x, y) in enumerate(zip(got, want[k])):
            assert_bits(x, y, f"DDP replay {k}, buffer {i}")
        del junk


@pytest.mark.parametrize("writes", [(0, 0), (64, 24)], ids=["chunk-writes", "clock-windows"])
def test_graph_replays_equal_eager_burst_steps(writes):
    """The P=64 step with the burst reduce (forced on a shard of about three
    chunks through the test build, writing g a chunk at a time or in short
    clock windows), shard-compact contributions, the bf16 parameters in shard
    layout, and the no-allocation reduce beside it, captured once and
    replayed."""
    import numpy as np
    P, r = 64, 9
    rng = np.random.default_rng(91)
    with G.test_hooks():
        G.set_reduce_path(G.REDUCE_PATH_BURST)
        G.set_burst_window(*writes)
        try:
            plan = G.Plan([int(2.6 * 32768) * P], 1 << 40, P, 8).upload()
            S = plan.shard_len
            hp = G.make_hp(lr=2e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=10)
            cs = [torch.from_numpy(rng.normal(0, 1e-3, S).astype(np.float32)).to(torch.bfloat16)
                  .view(torch.uint16).cuda() for _ in range(P)]
            ws = torch.zeros(G.workspace_bytes(S) // 8, dtype=torch.float64, device="cuda")

            def buffers():
                gen = torch.Generator(device="cuda").manual_seed(5)
                th = torch.randn(S, device="cuda", generator=gen) * 0.02
                m = torch.randn(S, device="cuda", generator=gen) * 1e-4
                v = (torch.randn(S, device="cuda", generator=gen) * 1e-6).abs()
                return dict(th=th, m=m, v=v, g=torch.empty(S, device="cuda"),
                            g2=torch.empty(S, device="cuda"),
                            parts=torch.full((P,), 0.25, dtype=torch.float64, device="cuda"),
                            p2=torch.zeros(1, dtype=torch.float64, device="cuda"),
                            coef=torch.empty(1, device="cuda"),
                            out=torch.zeros(S, dtype=torch.uint16, device="cuda"))

            def step(b):
                G.shard_reduce_mean(plan, r, cs, G.LAYOUT_SHARD_COMPACT, b["g"], b["parts"][r:r + 1], ws)
                G.shard_reduce_mean_noalloc(plan, r, cs, G.LAYOUT_SHARD_COMPACT, b["g2"], b["p2"])
                G.clip_coef(b["parts"], 1.0, b["coef"])
                G.shard_adamw_step(plan, r, b["th"], b["m"], b["v"], b["g"], b["coef"], hp, None, b["out"])

            def snapshot(b):
                torch.cuda.synchronize()
                return [host(b[k]) for k in ("g", "g2", "parts", "p2", "coef", "th", "m", "v", "out")]

            eager = buffers()
            want = []
            for _ in range(3):
                step(eager)
                want.append(snapshot(eager))
            assert_bits(want[0][1], want[0][0], "no-allocation g against the workspace form")
            b = buffers()
            torch.cuda.synchronize()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                step(b)
            torch.cuda.synchronize()
            for k in range(3):
                graph.replay()
                junk = torch.randn(1 << 20, device="cuda").sum()    # eager work between replays
                torch.cuda.synchronize()
                got = snapshot(b)
                for i, (x, y) in enumerate(zip(got, want[k])):
                    assert_bits(x, y, f"burst replay {k}, buffer {i}")
                del junk
        finally:
            G.set_reduce_path(G.REDUCE_PATH_BY_SIZE)
            G.set_burst_window(0, 0)
