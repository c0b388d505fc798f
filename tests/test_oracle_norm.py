"""Pins for the oracle's squared-norm partials and clip coefficient: exact
summation (math.fsum), closed forms, and PyTorch's clip_grad_norm_ (the
routine the page calls)."""
import math

import numpy as np
import torch

from oracle.norm import clip_coef, sqnorm_partial, total


def test_partial_matches_exact_sum():
    g = np.random.default_rng(2).normal(0, 3e-4, 1 << 18).astype(np.float32)
    exact = math.fsum(float(x) * float(x) for x in g)   # fp32 squares are exact in fp64
    assert abs(sqnorm_partial(g) - exact) <= 1e-14 * exact
    v = torch.linalg.vector_norm(torch.from_numpy(g).double()).item() ** 2
    assert abs(sqnorm_partial(g) - v) <= 1e-13 * v


def test_partial_closed_forms():
    a = np.float32(0.375)
    assert sqnorm_partial(np.full(1000, a, np.float32)) == 1000 * 0.375 ** 2
    assert sqnorm_partial(np.zeros(10, np.float32)) == 0.0
    assert sqnorm_partial(np.array([3, -4], np.float32)) == 25.0
    assert total([1.0, 2.0, 4.0]) == 7.0


def test_clip_matches_torch_clip_grad_norm():
    rng = np.random.default_rng(4)
    for scale in (1e-3, 0.05, 0.3, 1.0, 7.0):
        gs = [rng.normal(0, scale, n).astype(np.float32) for n in (100, 37, 1000)]
        T = total([sqnorm_partial(g) for g in gs])
        norm32, coef = clip_coef(T, 1.0)
        ts = [torch.nn.Parameter(torch.zeros(len(g))) for g in gs]
        for t, g in zip(ts, gs):
            t.grad = torch.from_numpy(g.copy())
        tn = torch.nn.utils.clip_grad_norm_(ts, 1.0)
        assert abs(float(tn) - float(norm32)) <= 2e-7 * float(norm32)
        for t, g in zip(ts, gs):
            np.testing.assert_allclose(t.grad.numpy(), g * coef, rtol=3e-7, atol=0)
        assert (coef == 1.0) == (float(norm32) + 1e-6 <= 1.0)


def test_clip_special_values():
    # one gradient element equal to 2 is scaled to 2/(2+1e-6) in fp32 (0.99999952)
    _, coef = clip_coef(4.0, 1.0)
    assert np.float32(2.0) * coef == np.float32(0.99999952)
    assert clip_coef(0.0, 1.0) == (0.0, 1.0)                # zero gradient: no scaling
    n, c = clip_coef(0.25, 1.0)
    assert n == 0.5 and c == 1.0
    n, c = clip_coef(1.0, 1.0)                              # exactly at the threshold: 1/(1+1e-6)
    assert n == 1.0 and c == np.float32(1.0) / (np.float32(1.0) + np.float32(1e-6)) and c < 1


def test_clip_propagates_nan_like_torch():
    n, c = clip_coef(float("nan"), 1.0)
    assert np.isnan(n) and np.isnan(c)
    t = torch.nn.Parameter(torch.zeros(2))
    t.grad = torch.tensor([float("nan"), 1.0])
    torch.nn.utils.clip_grad_norm_([t], 1.0)
    assert torch.isnan(t.grad).all()
