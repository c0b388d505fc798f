"""One synchronous data-parallel step, composed from the oracle's parts.

ZeRO-1/2 ("Data Parallelism: DDP, ZeRO and FSDP", section "The three stages"):
reduce-scatter the gradients, clip with the global norm, update the owned
shard, all-gather the updated bf16 parameters.  DDP / NO_SHARD ("Data
parallelism in depth" §4.1 and §6.3): all-reduce the gradients, every rank
updates the whole model.  "Data Parallelism: From Parameter Server to Ring
All-Reduce" §1 and §10: the replicas stay identical because each rank applies an identical update.
"""
from __future__ import annotations

import numpy as np

from .adamw import adamw
from .layout import ag_write
from .norm import clip_coef, sqnorm_partial, total
from .pack import owner_view
from .reduce import reduce_mean, ring_allreduce_sim


def _hp(hp):
    return dict(lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps,
                weight_decay=hp.weight_decay, step=hp.step)


def zero_step_all_owners(plan, flats, theta_full, m_full, v_full, hp):
    """Every owner's shard step.  flats[q]: rank q's packed bf16 gradients;
    *_full: flat fp32 optimizer state (each owner reads its own chunks)."""
    P = plan.world_size
    gs = [reduce_mean([owner_view(plan, f, r) for f in flats], r) for r in range(P)]
    partials = [sqnorm_partial(g) for g in gs]
    T = total(partials)
    norm32, coef = clip_coef(T, hp.max_norm)
    outs = []
    gathered = np.zeros(plan.flat_len, dtype=np.uint16)
    for r in range(P):
        th, m1, v1, p = adamw(owner_view(plan, theta_full, r), owner_view(plan, m_full, r),
                              owner_view(plan, v_full, r), gs[r], coef, **_hp(hp))
        outs.append((th, m1, v1, p))
        ag_write(plan, r, p, gathered)
    return dict(g=gs, partials=partials, total=T, norm=norm32, coef=coef,
                theta=[o[0] for o in outs], m=[o[1] for o in outs],
                v=[o[2] for o in outs], p=[o[3] for o in outs], gathered=gathered)


def ddp_step(plan, flats, theta_full, m_full, v_full, hp):
    """Unsharded reference: ring all-reduce, one global norm, AdamW on all."""
    results, rs_sent, ag_sent = ring_allreduce_sim(plan, flats)
    g = results[0]
    T = sqnorm_partial(g)
    norm32, coef = clip_coef(T, hp.max_norm)
    th, m1, v1, p = adamw(theta_full, m_full, v_full, g, coef, **_hp(hp))
    return dict(g=g, replicas=results, total=T, norm=norm32, coef=coef,
                theta=th, m=m1, v=v1, p=p, rs_sent=rs_sent, ag_sent=ag_sent)
