"""Mixed-precision AdamW update of one shard, in a fixed fp32 operation order.

The pages call the optimizer without printing it: AdamW(lr=2e-4,
weight_decay=0.1) ("Distributed Training: Data Parallel, Model Parallel and
FSDP Strategies", section "Inside DDP: Bucketed All-Reduce, Gradient
Synchronization and Overlap"), with fp32 master weights, fp32 first and second
moments and bf16 working parameters ("Data Parallelism: DDP, ZeRO and FSDP",
section "The memory ledger"; "Data parallelism in depth" §7).  ZeRO-1/2 run
this update only on the shard a rank owns ("Data Parallelism: DDP, ZeRO and
FSDP", section "The three stages").

AdamW, with decoupled weight decay applied to the old weights and eps outside
the square root, for step t (the plainest reading of the optimizer the page
calls):
    g  <- g * coef                                   (clip)
    m  <- b1*m + (1-b1)*g
    v  <- b2*v + (1-b2)*g*g
    mh <- m / (1-b1^t);  vh <- v / (1-b2^t)
    u  <- mh / (sqrt(vh) + eps)
    theta <- theta*(1 - lr*wd) - lr*u
    p  <- bf16(theta)

Every operation below is one NumPy ufunc on float32 (one IEEE rounding each,
no fused multiply-add).  The scalars 1-b1, 1-b2, 1-b1^t, 1-b2^t and 1-lr*wd are
formed in float64 from the hyperparameters and rounded once to float32.
"""
from __future__ import annotations

import numpy as np

from .bf16 import narrow


def scalars(lr, beta1, beta2, eps, weight_decay, step):
    """The fp32 constants of the update, each rounded once from float64."""
    if step < 1:
        raise ValueError("step must be >= 1")
    f = np.float32
    return dict(b1=f(beta1), omb1=f(1.0 - beta1), b2=f(beta2), omb2=f(1.0 - beta2),
                bc1=f(1.0 - beta1 ** step), bc2=f(1.0 - beta2 ** step),
                lr=f(lr), eps=f(eps), decay=f(1.0 - lr * weight_decay))


def adamw(theta, m, v, g, coef, lr, beta1, beta2, eps, weight_decay, step):
    """Returns (theta', m', v', p_bf16) for float32 arrays theta, m, v, g."""
    s = scalars(lr, beta1, beta2, eps, weight_decay, step)
    theta = np.asarray(theta, dtype=np.float32)
    m = np.asarray(m, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    gc = g * np.float32(coef)
    m1 = (s["b1"] * m) + (s["omb1"] * gc)
    v1 = (s["b2"] * v) + (s["omb2"] * (gc * gc))
    mh = m1 / s["bc1"]
    vh = v1 / s["bc2"]
    u = mh / (np.sqrt(vh) + s["eps"])
    th = (theta * s["decay"]) - (s["lr"] * u)
    return th.astype(np.float32), m1.astype(np.float32), v1.astype(np.float32), narrow(th)
