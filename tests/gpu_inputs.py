"""Device-side input assembly for the HIP path: the same seeded values as
tests/oracle_inputs.py, generated on the GPU and placed with the library's own
plan (never the oracle's)."""
from __future__ import annotations

import torch

from synth import gen
from synth import workloads as W

STATE_KINDS = ((W.KIND_MASTER, W.MASTER_STD, gen.MODE_F32),
               (W.KIND_EXP_AVG, W.EXP_AVG_STD, gen.MODE_F32),
               (W.KIND_EXP_AVG_SQ, W.EXP_AVG_SQ_STD, gen.MODE_ABS))


def prefix(numel):
    out, s = [], 0
    for n in numel:
        out.append(s)
        s += n
    return out


def rank_grads(w, q, out=None):
    """Rank q's gradients as one forward-order device buffer plus per-tensor views."""
    if out is None:
        out = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
    gen.dev_fill(out, w.cfg_id, W.KIND_GRAD, q, 0, w.grad_std, gen.MODE_BF16)
    views = [out[s:s + n] for s, n in zip(prefix(w.numel), w.numel)]
    return out, views


def rank_grads_separate(w, q):
    """Rank q's gradients as separate allocations (one per tensor)."""
    pre = prefix(w.numel)
    ts = []
    for s, n in zip(pre, w.numel):
        t = torch.empty(n, dtype=torch.uint16, device="cuda")
        if n:
            gen.dev_fill(t, w.cfg_id, W.KIND_GRAD, q, s, w.grad_std, gen.MODE_BF16)
        ts.append(t)
    return ts


def owner_pieces(plan, w, r):
    """(shard offset, parameter index, length) of owner r's parameter pieces,
    from the library plan's tables."""
    pre = prefix(w.numel)
    pieces = []
    for b in plan.buckets():
        cs = b["base"] + r * b["chunk"]
        ce = cs + b["chunk"]
        for k in range(b["n_tensors"]):
            t = b["first_tensor"] - k
            ts = plan.tensor(t)[0]
            te = ts + w.numel[t]
            s, e = max(cs, ts), min(ce, te)
            if s < e:
                pieces.append((b["shard_off"] + (s - cs), pre[t] + (s - ts), e - s))
    return pieces


def fill_pieces(out, pieces, w, kind, rank, std, mode):
    gen.dev_fill_pieces(out, pieces, w.cfg_id, kind, rank, std, mode)


def owner_state(plan, w, r):
    """master, m, v of owner r's shard (pads zero)."""
    pieces = owner_pieces(plan, w, r)
    out = []
    for kind, std, mode in STATE_KINDS:
        t = torch.zeros(plan.shard_len, dtype=torch.float32, device="cuda")
        fill_pieces(t, pieces, w, kind, 0, std, mode)
        out.append(t)
    return out


def compact_contribs(plan, w, r):
    """The shard_len gradients each rank q sends to owner r (shard layout)."""
    pieces = owner_pieces(plan, w, r)
    out = []
    for q in range(w.world_size):
        t = torch.zeros(plan.shard_len, dtype=torch.uint16, device="cuda")
        fill_pieces(t, pieces, w, W.KIND_GRAD, q, w.grad_std, gen.MODE_BF16)
        out.append(t)
    return out


def full_state(plan, w):
    """master, m, v over the whole bucket-major flat buffer (the replicated
    DDP state), pads zero, placed with the library plan's tensor offsets."""
    pre = prefix(w.numel)
    out = []
    for kind, std, mode in STATE_KINDS:
        t = torch.zeros(plan.flat_len, dtype=torch.float32, device="cuda")
        for ti, n in enumerate(w.numel):
            if n:
                off = plan.tensor(ti)[0]
                gen.dev_fill(t[off:off + n], w.cfg_id, kind, 0, pre[ti], std, mode)
        out.append(t)
    return out
