"""Pack per-tensor gradients into the bucket-major flat buffer, and back.

"Data parallelism in depth" §4.2 (The Bucket mechanism) packs the gradients of
several parameters into one bucket so that one collective serves them all;
"Distributed Training: Data Parallel, Model Parallel and FSDP Strategies",
section "Inside DDP", notes the buckets can be the gradients' own storage
(gradient_as_bucket_view).  The flat buffer holds bucket b at [base_b, base_b+L_b):
its tensors densely in bucket order, then zeros up to L_b.
"""
from __future__ import annotations

import numpy as np

from .plan import Plan


def pack(plan: Plan, grads, dtype=np.uint16) -> np.ndarray:
    """grads: list (forward order) of 1-D arrays (bf16 bits as uint16 by default)
    -> flat[flat_len] of the same dtype, pads zero."""
    flat = np.zeros(plan.flat_len, dtype=dtype)
    for t, g in enumerate(grads):
        g = np.asarray(g, dtype=dtype).reshape(-1)
        if g.size != plan.numel[t]:
            raise ValueError(f"tensor {t}: {g.size} elements, plan says {plan.numel[t]}")
        off = plan.tensor_offset[t]
        flat[off:off + g.size] = g
    return flat


def unpack(plan: Plan, flat: np.ndarray):
    """Inverse of pack: the per-tensor views of a flat buffer (forward order)."""
    return [flat[plan.tensor_offset[t]:plan.tensor_offset[t] + n].copy()
            for t, n in enumerate(plan.numel)]


def owner_view(plan: Plan, flat: np.ndarray, r: int) -> np.ndarray:
    """Rank r's chunks of a flat buffer, concatenated in bucket order (shard layout)."""
    parts = [flat[slice(*plan.chunk_range(b, r))] for b in range(len(plan.buckets))]
    if not parts:
        return flat[:0].copy()
    return np.concatenate(parts)


def accumulate(plan: Plan, flat: np.ndarray, grads) -> np.ndarray:
    """Gradient accumulation into the bucket buffer between synchronisations.

    "Distributed Training: Data Parallel, Model Parallel and FSDP Strategies",
    section "Selecting and Tuning Your Strategy" (no_sync code): gradients of
    micro-batches that skip synchronisation accumulate, and only the last
    micro-batch synchronises.  With gradient_as_bucket_view (section "Inside
    DDP") the gradients are views of the bucket buffer, so each backward adds
    into it in the gradient dtype: flat = bf16(f32(flat) + f32(grad)), one
    round to nearest even per addition.  Pads are untouched.  Returns a new
    array.
    """
    from .bf16 import narrow, widen
    out = np.array(flat, dtype=np.uint16, copy=True)
    for t, g in enumerate(grads):
        g = np.asarray(g, dtype=np.uint16).reshape(-1)
        if g.size != plan.numel[t]:
            raise ValueError(f"tensor {t}: {g.size} elements, plan says {plan.numel[t]}")
        off = plan.tensor_offset[t]
        out[off:off + g.size] = narrow(widen(out[off:off + g.size]) + widen(g))
    return out


def pack_f32(plan: Plan, grads) -> np.ndarray:
    """First micro-batch of an fp32 accumulation: the bf16 gradients widened
    (exactly) into an fp32 bucket-major buffer, pads zero.

    Gradient accumulation between synchronisations ("Distributed Training: Data
    Parallel, Model Parallel and FSDP Strategies", section "Selecting and Tuning
    Your Strategy", the no_sync loop) with the reduction dtype fp32 (same page,
    section "FSDP1 vs FSDP2 and DTensor", reduce_dtype = fp32): the buckets hold
    fp32 sums of the micro-batches' bf16 gradients.
    """
    from .bf16 import widen
    flat = np.zeros(plan.flat_len, dtype=np.float32)
    for t, g in enumerate(grads):
        g = np.asarray(g, dtype=np.uint16).reshape(-1)
        if g.size != plan.numel[t]:
            raise ValueError(f"tensor {t}: {g.size} elements, plan says {plan.numel[t]}")
        off = plan.tensor_offset[t]
        flat[off:off + g.size] = widen(g)
    return flat


def accumulate_f32(plan: Plan, flat32: np.ndarray, grads) -> np.ndarray:
    """Later micro-batches of the fp32 accumulation (passages as for pack_f32):
    flat32 = flat32 + f32(grad), one fp32 addition (round to nearest even) per
    element; pads untouched.  Returns a new array."""
    from .bf16 import widen
    out = np.array(flat32, dtype=np.float32, copy=True)
    for t, g in enumerate(grads):
        g = np.asarray(g, dtype=np.uint16).reshape(-1)
        if g.size != plan.numel[t]:
            raise ValueError(f"tensor {t}: {g.size} elements, plan says {plan.numel[t]}")
        off = plan.tensor_offset[t]
        out[off:off + g.size] = out[off:off + g.size] + widen(g)
    return out
