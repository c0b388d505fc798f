"""All-gather layout of the updated bf16 parameters.

"Data Parallelism: DDP, ZeRO and FSDP", section "The three stages": under
ZeRO-1/2 each rank updates its own shard, and an all-gather then gives every
rank all of the new parameters.  "Data Parallelism: From Parameter Server to
Ring All-Reduce" §5: after the all-gather each rank has the whole tensor, with
chunk c back at position c.  So
rank r's updated chunk of bucket b sits at flat [base_b + r*C_b, +C_b) of the
gathered bucket-major buffer.
"""
from __future__ import annotations

import numpy as np

from .plan import Plan


def ag_write(plan: Plan, r: int, shard: np.ndarray, gathered: np.ndarray) -> None:
    """Writes rank r's shard-layout values into the gathered flat buffer."""
    for b, bk in enumerate(plan.buckets):
        s, e = plan.chunk_range(b, r)
        gathered[s:e] = shard[bk.shard_off: bk.shard_off + bk.chunk]


def ag_read(plan: Plan, r: int, gathered: np.ndarray) -> np.ndarray:
    """Rank r's chunks read back out of a gathered flat buffer (shard layout)."""
    parts = [gathered[slice(*plan.chunk_range(b, r))] for b in range(len(plan.buckets))]
    return np.concatenate(parts) if parts else gathered[:0].copy()
