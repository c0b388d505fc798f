"""Oracle-side input assembly: seeded values from the host generator placed
with the oracle's own plan.  Used by the CPU pins and by the GPU parity tests
(the GPU side assembles the same values with the library's plan)."""
from __future__ import annotations

import numpy as np

from oracle import pack as opack
from synth import gen
from synth import workloads as W


def prefix(numel):
    out, s = [], 0
    for n in numel:
        out.append(s)
        s += n
    return out


def rank_grads(w, q):
    """Rank q's per-tensor bf16 gradients (forward order), keyed by parameter index."""
    flat = gen.host_fill(w.cfg_id, W.KIND_GRAD, q, 0, w.n_params, w.grad_std, gen.MODE_BF16)
    pre = prefix(w.numel)
    return [flat[s:s + n] for s, n in zip(pre, w.numel)]


def rank_flat(plan, w, q):
    return opack.pack(plan, rank_grads(w, q))


STATE_KINDS = ((W.KIND_MASTER, W.MASTER_STD, gen.MODE_F32),
               (W.KIND_EXP_AVG, W.EXP_AVG_STD, gen.MODE_F32),
               (W.KIND_EXP_AVG_SQ, W.EXP_AVG_SQ_STD, gen.MODE_ABS))


def full_state(plan, w):
    """Flat fp32 (master, m, v) over the whole bucket-major buffer, pads zero."""
    out = []
    for kind, std, mode in STATE_KINDS:
        vals = gen.host_fill(w.cfg_id, kind, 0, 0, w.n_params, std, mode)
        pre = prefix(w.numel)
        out.append(opack.pack(plan, [vals[s:s + n] for s, n in zip(pre, w.numel)],
                              dtype=np.float32))
    return out


def owner_pieces(plan, r):
    """(shard offset, parameter index, length) pieces of owner r's shard that
    hold parameters (pads are not covered)."""
    pre = prefix(plan.numel)
    pieces = []
    for b, bk in enumerate(plan.buckets):
        cs, ce = plan.chunk_range(b, r)
        for t in bk.tensors:
            ts, te = plan.tensor_offset[t], plan.tensor_offset[t] + plan.numel[t]
            s, e = max(cs, ts), min(ce, te)
            if s < e:
                pieces.append((bk.shard_off + (s - cs), pre[t] + (s - ts), e - s))
    return pieces


def shard_param_index(plan, r):
    """For each element of owner r's shard: its parameter index, or -1 for a pad."""
    idx = np.full(plan.shard_len, -1, dtype=np.int64)
    for so, pi, n in owner_pieces(plan, r):
        idx[so:so + n] = np.arange(pi, pi + n, dtype=np.int64)
    return idx


def values_at(w, kind, rank, std, mode, param_idx):
    """Generator values at the given parameter indices; zero where index < 0."""
    dtype = np.uint16 if mode == gen.MODE_BF16 else np.float32
    out = np.zeros(param_idx.size, dtype=dtype)
    ok = param_idx >= 0
    if ok.any():
        out[ok] = gen.host_fill_idx(w.cfg_id, kind, rank, param_idx[ok], std, mode)
    return out


def param_index_of_flat(plan, flat_pos):
    """Parameter index (forward-order concatenation) of flat positions; -1 for pads."""
    flat_pos = np.asarray(flat_pos, dtype=np.int64)
    order = [t for bk in plan.buckets for t in bk.tensors]      # increasing flat offset
    offs = np.array([plan.tensor_offset[t] for t in order], dtype=np.int64)
    ns = np.array([plan.numel[t] for t in order], dtype=np.int64)
    pre = np.array(prefix(plan.numel), dtype=np.int64)
    pres = np.array([pre[t] for t in order], dtype=np.int64)
    k = np.searchsorted(offs, flat_pos, side="right") - 1
    ok = k >= 0
    kk = np.where(ok, k, 0)
    inside = ok & (flat_pos < offs[kk] + ns[kk])
    return np.where(inside, pres[kk] + (flat_pos - offs[kk]), -1)


def flat_pos_of_shard(plan, r, shard_idx):
    """Flat (and all-gather) position of owner r's shard indices."""
    shard_idx = np.asarray(shard_idx, dtype=np.int64)
    so = np.array([bk.shard_off for bk in plan.buckets], dtype=np.int64)
    base = np.array([bk.base for bk in plan.buckets], dtype=np.int64)
    ch = np.array([bk.chunk for bk in plan.buckets], dtype=np.int64)
    # the last bucket whose chunk starts at or before i (empty chunks are skipped)
    b = np.searchsorted(so, shard_idx, side="right") - 1
    return base[b] + r * ch[b] + (shard_idx - so[b])
