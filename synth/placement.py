"""Device-side input assembly: the seeded values of synth.gen placed in HBM with
the library's own plan tables (never the oracle's).

Every buffer is filled with one launch (a table of pieces {destination,
parameter index, length}), so a benchmark or a profiled command issues a few
dozen fill launches in all; gen.fill_launches counts them.  This module holds
none of the method's arithmetic: it decides where each seeded value goes.
"""
from __future__ import annotations

import torch

from . import gen
from . import workloads as W

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
    """Rank q's gradients as one forward-order device buffer (one launch) plus
    per-tensor views of it."""
    if out is None:
        out = torch.empty(w.n_params, dtype=torch.uint16, device="cuda")
    gen.dev_fill(out, w.cfg_id, W.KIND_GRAD, q, 0, w.grad_std, gen.MODE_BF16)
    views = [out[s:s + n] for s, n in zip(prefix(w.numel), w.numel)]
    return out, views


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


def fill_pieces(out, pieces, w, kind, rank, std, mode, interleave=None):
    gen.dev_fill_pieces(out, pieces, w.cfg_id, kind, rank, std, mode, interleave=interleave)


def owner_state(plan, w, r):
    """master, m, v of owner r's shard (pads zero), one launch each."""
    pieces = owner_pieces(plan, w, r)
    out = []
    for kind, std, mode in STATE_KINDS:
        t = torch.zeros(plan.shard_len, dtype=torch.float32, device="cuda")
        fill_pieces(t, pieces, w, kind, 0, std, mode)
        out.append(t)
    return out


def compact_contribs(plan, w, r):
    """The shard_len gradients each rank q sends to owner r (shard layout),
    one buffer and one launch per rank."""
    pieces = owner_pieces(plan, w, r)
    out = []
    for q in range(w.world_size):
        t = torch.zeros(plan.shard_len, dtype=torch.uint16, device="cuda")
        fill_pieces(t, pieces, w, W.KIND_GRAD, q, w.grad_std, gen.MODE_BF16)
        out.append(t)
    return out


def interleaved_contribs(plan, w, r, interleaved_len):
    """The same values as compact_contribs in one rank-interleaved receive
    buffer of interleaved_len elements (rank q's values for shard elements
    [512t, 512t + 512) at (t*P + q)*512); one launch per rank.  Pads and the
    unused tails of the last tile's pieces are zero."""
    pieces = owner_pieces(plan, w, r)
    P = w.world_size
    buf = torch.zeros(interleaved_len, dtype=torch.uint16, device="cuda")
    for q in range(P):
        fill_pieces(buf, pieces, w, W.KIND_GRAD, q, w.grad_std, gen.MODE_BF16, interleave=(P, q))
    return buf


def full_state(plan, w):
    """master, m, v over the whole bucket-major flat buffer (the replicated
    DDP state), pads zero, placed with the library plan's tensor offsets; one
    launch each."""
    pieces = [(plan.tensor(t)[0], s, n) for t, (s, n) in enumerate(zip(prefix(w.numel), w.numel))
              if n]
    out = []
    for kind, std, mode in STATE_KINDS:
        t = torch.zeros(plan.flat_len, dtype=torch.float32, device="cuda")
        fill_pieces(t, pieces, w, kind, 0, std, mode)
        out.append(t)
    return out
