"""Global gradient L2 norm and the clip coefficient for clipping at 1.0.

"Distributed Training: Data Parallel, Model Parallel and FSDP Strategies",
section "Inside DDP: Bucketed All-Reduce, Gradient Synchronization and
Overlap": after the averaged gradients are ready, clip_grad_norm_(params, 1.0)
runs before optimizer.step().  The norm is the L2 norm of the whole reduced
gradient, so under sharding each rank forms the squared-norm partial of the
shard it owns and the partials are summed.

Readings: partials are exact squares of fp32 values summed in fp64; the P
partials are added in rank order; the norm is sqrt in fp64 rounded once to
fp32; the coefficient is min(1, max_norm / (norm + 1e-6)) in fp32, the form of
PyTorch's clip_grad_norm_ that the page calls (a NaN norm gives a NaN
coefficient, as its clamp does); the gradient is then scaled by
the coefficient (a multiply by exactly 1 when no clipping happens).
"""
from __future__ import annotations

import math

import numpy as np


def sqnorm_partial(g: np.ndarray) -> float:
    """Sum of squares of an fp32 shard, in fp64."""
    g64 = np.asarray(g, dtype=np.float32).astype(np.float64)
    return float(np.sum(g64 * g64))


def total(partials) -> float:
    """Partials of ranks 0..P-1 added in rank order (fp64)."""
    t = 0.0
    for p in partials:
        t = t + float(p)
    return t


def clip_coef(total_sq: float, max_norm: float = 1.0):
    """Returns (norm32, coef32)."""
    norm32 = np.float32(math.sqrt(total_sq))
    c = np.float32(max_norm) / (norm32 + np.float32(1e-6))
    coef32 = np.minimum(np.float32(1.0), np.float32(c))   # NaN propagates, as in torch.clamp
    return np.float32(norm32), coef32
