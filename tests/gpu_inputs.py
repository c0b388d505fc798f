"""Device-side input assembly for the GPU tests: synth.placement (the same
seeded values as tests/oracle_inputs.py, placed with the library's own plan),
plus per-tensor allocations for the tests that want separate buffers."""
from __future__ import annotations

import torch

from synth import gen
from synth import workloads as W
from synth.placement import (STATE_KINDS, compact_contribs, fill_pieces, full_state,  # noqa: F401
                             interleaved_contribs, owner_pieces, owner_state, prefix, rank_grads)


def rank_grads_separate(w, q):
    """Rank q's gradients as separate allocations, one fill launch per tensor
    (tests only: benchmarks and profiled commands place inputs with one launch
    per buffer)."""
    pre = prefix(w.numel)
    ts = []
    for s, n in zip(pre, w.numel):
        t = torch.empty(n, dtype=torch.uint16, device="cuda")
        if n:
            gen.dev_fill(t, w.cfg_id, W.KIND_GRAD, q, s, w.grad_std, gen.MODE_BF16)
        ts.append(t)
    return ts
