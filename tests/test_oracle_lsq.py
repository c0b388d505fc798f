"""Pins for oracle/lsq.py, the least-squares model behind the gradient-mean
check ("Data parallelism in depth" §2, Mathematical foundation of data
parallelism: each rank's gradient is its shard's locally averaged gradient,
and their average is the full-batch gradient).

The oracle computes gradients sample by sample.  The pins here never
differentiate by hand: they evaluate the LOSS, (1/B) sum_i 1/2 (x_i . theta -
y_i)^2, in exact rationals and take the central difference
(L(theta + e_j) - L(theta - e_j)) / 2, which is the exact partial derivative
of a quadratic.  A second pin is the integer matrix form X^T (X theta - y) / B
(NumPy int64, not the oracle's loop), and a third a hand-worked example.  A
flipped residual sign, a dropped x factor, a sum in place of the mean, or a
shard that is not the k-th contiguous block each fail them (planted below).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import lsq
from synth import workloads as W


def loss(X, theta, Y):
    """(1/B) sum_i 1/2 (x_i . theta - y_i)^2 in exact rationals."""
    tot = Fraction(0)
    for x, y in zip(X, Y):
        r = sum(Fraction(int(a)) * Fraction(b) for a, b in zip(x, theta)) - int(y)
        tot += Fraction(1, 2) * r * r
    return tot / len(X)


def central_difference_grad(X, theta, Y):
    """Exact gradient of the quadratic loss: step 1 on each coordinate."""
    out = []
    for j in range(len(theta)):
        up = [Fraction(int(t)) + (1 if k == j else 0) for k, t in enumerate(theta)]
        dn = [Fraction(int(t)) - (1 if k == j else 0) for k, t in enumerate(theta)]
        out.append((loss(X, up, Y) - loss(X, dn, Y)) / 2)
    return out


def matrix_grad(X, theta, Y):
    """X^T (X theta - y) / B with integer matrices."""
    X = np.asarray(X, dtype=np.int64)
    r = X @ np.asarray(theta, dtype=np.int64) - np.asarray(Y, dtype=np.int64)
    return [Fraction(int(v), len(X)) for v in X.T @ r]


def shard_pins(X, theta, Y, N):
    """Rank k's pin: the central difference of the k-th contiguous block's own
    mean loss."""
    per = len(X) // N
    return [central_difference_grad(X[k * per:(k + 1) * per], theta, Y[k * per:(k + 1) * per])
            for k in range(N)]


def pinned(full_fn, shard_fn, problems):
    """True if full_fn and shard_fn agree with every pin on every problem."""
    for X, theta, Y, N in problems:
        full = full_fn(X, theta, Y)
        if full != central_difference_grad(X, theta, Y) or full != matrix_grad(X, theta, Y):
            return False
        if shard_fn(X, theta, Y, N) != shard_pins(X, theta, Y, N):
            return False
    return True


def problems():
    X, theta, Y = W.lsq_problem()
    rng = np.random.default_rng(2)
    out = [(X, theta, Y, 4)]
    for B, F, N in ((12, 3, 3), (8, 5, 2), (20, 2, 5)):
        out.append((rng.integers(-3, 4, size=(B, F)), rng.integers(-2, 3, size=F),
                    rng.integers(-4, 5, size=B), N))
    return out


def test_hand_worked_example():
    # x1 = (1, 2), y1 = 0 and x2 = (3, -1), y2 = 1 at theta = (1, 0):
    # residuals 1 and 2, per-sample gradients (1, 2) and (6, -2), mean (7/2, 0).
    X, theta, Y = [[1, 2], [3, -1]], [1, 0], [0, 1]
    assert lsq.sample_grad(X[0], theta, Y[0]) == [1, 2]
    assert lsq.sample_grad(X[1], theta, Y[1]) == [6, -2]
    assert lsq.full_batch_grad(X, theta, Y) == [Fraction(7, 2), 0]
    # two ranks of one sample each: their local means are the per-sample gradients
    assert lsq.shard_grads(X, theta, Y, 2) == [[1, 2], [6, -2]]


def test_full_batch_and_shard_gradients_match_the_loss():
    assert pinned(lsq.full_batch_grad, lsq.shard_grads, problems())


def test_the_pins_agree_with_each_other():
    for X, theta, Y, _ in problems():
        assert central_difference_grad(X, theta, Y) == matrix_grad(X, theta, Y)


def test_shards_need_equal_local_batches():
    X, theta, Y = W.lsq_problem()
    with pytest.raises(ValueError):
        lsq.shard_grads(X, theta, Y, 5)


def _sample_grad_sign_flip(x, theta, y):
    r = int(y) - sum(int(a) * int(b) for a, b in zip(x, theta))
    return [Fraction(r * int(a)) for a in x]


def _sample_grad_no_x(x, theta, y):
    r = sum(int(a) * int(b) for a, b in zip(x, theta)) - int(y)
    return [Fraction(r)] * len(x)


def _sample_grad_x_squared(x, theta, y):
    r = sum(int(a) * int(b) for a, b in zip(x, theta)) - int(y)
    return [Fraction(r * int(a) * int(a)) for a in x]


def _shard_grads_summed(X, theta, Y, N):
    per = len(X) // N
    return [[s * per for s in g] for g in lsq.shard_grads(X, theta, Y, N)]


def _shard_grads_strided(X, theta, Y, N):
    idx = [list(range(k, len(X), N)) for k in range(N)]
    return [lsq.full_batch_grad([X[i] for i in ix], theta, [Y[i] for i in ix]) for ix in idx]


def _full_batch_sum(X, theta, Y):
    return [g * len(X) for g in lsq.full_batch_grad(X, theta, Y)]


@pytest.mark.parametrize("mutant", ["sign_flip", "no_x", "x_squared", "shard_sum",
                                    "shard_strided", "full_sum"])
def test_planted_mistakes_fail_the_pins(mutant, monkeypatch):
    full_fn, shard_fn = lsq.full_batch_grad, lsq.shard_grads
    if mutant == "sign_flip":
        monkeypatch.setattr(lsq, "sample_grad", _sample_grad_sign_flip)
    elif mutant == "no_x":
        monkeypatch.setattr(lsq, "sample_grad", _sample_grad_no_x)
    elif mutant == "x_squared":
        monkeypatch.setattr(lsq, "sample_grad", _sample_grad_x_squared)
    elif mutant == "shard_sum":
        shard_fn = _shard_grads_summed
    elif mutant == "shard_strided":
        shard_fn = _shard_grads_strided
    else:
        full_fn = _full_batch_sum
    assert not pinned(full_fn, shard_fn, problems())
