"""Least-squares model for the gradient-mean equivalence.

"Data parallelism in depth" §2 (Mathematical foundation of data parallelism):
with loss L = (1/B) sum_i l(x_i; theta) and the B samples split evenly over N
ranks, rank k's local gradient g_k = (N/B) sum_{i in D_k} grad l(x_i) and the
average of the g_k equals the full-batch gradient exactly.  "Data Parallelism:
DDP, ZeRO and FSDP", section "DDP, and why it works", states the same.

Here l(x; theta) = 1/2 (x . theta - y)^2, so grad l = (x . theta - y) x.
Computed with exact rationals.
"""
from __future__ import annotations

from fractions import Fraction


def sample_grad(x, theta, y):
    r = sum(int(a) * int(b) for a, b in zip(x, theta)) - int(y)
    return [Fraction(r * int(a)) for a in x]


def full_batch_grad(X, theta, Y):
    B = len(X)
    acc = [Fraction(0)] * len(theta)
    for x, y in zip(X, Y):
        acc = [a + s for a, s in zip(acc, sample_grad(x, theta, y))]
    return [a / B for a in acc]


def shard_grads(X, theta, Y, N):
    """Rank k's locally averaged gradient on the k-th contiguous shard."""
    B = len(X)
    if B % N:
        raise ValueError("the equivalence needs equal local batches")
    per = B // N
    out = []
    for k in range(N):
        acc = [Fraction(0)] * len(theta)
        for i in range(k * per, (k + 1) * per):
            acc = [a + s for a, s in zip(acc, sample_grad(X[i], theta, Y[i]))]
        out.append([Fraction(N, B) * a for a in acc])
    return out
