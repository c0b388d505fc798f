"""Pins for the oracle's AdamW: closed-form special cases, PyTorch's AdamW
(the optimizer the page calls; it pins the formula, to an absolute tolerance,
not the rounding of each step), and planted mistakes that the pins must catch."""
import numpy as np
import pytest
import torch

import oracle.adamw as oa
from synth.workloads import AdamWHP

HP = AdamWHP()


def run(theta, m, v, g, coef=np.float32(1), **kw):
    h = dict(lr=HP.lr, beta1=HP.beta1, beta2=HP.beta2, eps=HP.eps,
             weight_decay=HP.weight_decay, step=HP.step)
    h.update(kw)
    return oa.adamw(theta, m, v, g, coef, **h)


def state(n, seed=0, gstd=1e-3):
    r = np.random.default_rng(seed)
    f = np.float32
    return (r.normal(0, 0.02, n).astype(f), r.normal(0, 1e-4, n).astype(f),
            np.abs(r.normal(0, 1e-6, n)).astype(f), r.normal(0, gstd, n).astype(f))


def torch_adamw(theta, m, v, g, coef, lr=HP.lr, betas=(HP.beta1, HP.beta2), eps=HP.eps,
                wd=HP.weight_decay, step=HP.step, foreach=False):
    p = torch.nn.Parameter(torch.from_numpy(theta.copy()))
    opt = torch.optim.AdamW([p], lr=lr, betas=betas, eps=eps, weight_decay=wd, foreach=foreach)
    p.grad = torch.from_numpy(g.copy()) * float(coef)
    opt.step()                                           # creates the state
    with torch.no_grad():
        p.copy_(torch.from_numpy(theta))
    st = opt.state[p]
    st["exp_avg"].copy_(torch.from_numpy(m))
    st["exp_avg_sq"].copy_(torch.from_numpy(v))
    st["step"].fill_(step - 1)                           # this update uses exponent `step`
    p.grad = torch.from_numpy(g.copy()) * torch.tensor(coef, dtype=torch.float32)
    opt.step()
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def test_zero_learning_rate_keeps_theta_bitwise():
    th, m, v, g = state(5000)
    th1, m1, v1, _ = run(th, m, v, g, lr=0.0)
    assert np.array_equal(th1.view(np.uint32), th.view(np.uint32))
    assert not np.array_equal(m1, m)


def test_zero_gradient_and_moments_give_pure_decay():
    th = state(5000)[0]
    z = np.zeros_like(th)
    th1, m1, v1, p = run(th, z, z, z)
    decay = np.float32(1.0 - HP.lr * HP.weight_decay)
    assert np.array_equal(th1, th * decay) and not (m1.any() or v1.any())


def test_first_step_is_sign_descent():
    # t=1, m=v=0, wd=0: mh = g, vh = g^2, so the step is lr * g/(|g| + eps)
    th, _, _, g = state(5000, gstd=1e-2)
    z = np.zeros_like(th)
    th1, m1, v1, _ = run(th, z, z, g, weight_decay=0.0, step=1)
    g64 = g.astype(np.float64)
    want = th.astype(np.float64) - HP.lr * g64 / (np.abs(g64) + HP.eps)
    np.testing.assert_allclose(th1, want, rtol=0, atol=4e-9)
    assert np.abs(th1 - (th - np.float32(HP.lr) * np.sign(g))).max() > 1e-8   # eps is visible
    np.testing.assert_allclose(m1, np.float32(1 - HP.beta1) * g, rtol=1e-7)


@pytest.mark.parametrize("gstd,coef,vscale", [(1e-3, 1.0, 1.0), (1e-3, 0.0345, 1.0),
                                               (0.1, 0.0196, 1.0), (1e-5, 1.0, 1e-8)])
@pytest.mark.parametrize("foreach", [False, True])
def test_matches_torch_adamw(gstd, coef, vscale, foreach):
    th, m, v, g = state(20000, seed=9, gstd=gstd)
    v = (v * np.float32(vscale)).astype(np.float32)
    c = np.float32(coef)
    th1, m1, v1, p = run(th, m, v, g, c)
    tth, tm, tv = torch_adamw(th, m, v, g, c, foreach=foreach)
    assert torch_pin_ok((th1, m1, v1), (tth, tm, tv))


# The pin's tolerances (absolute plus relative: torch orders the operations
# differently, so it fixes the formula, not each rounding).  The planted
# mistakes below are judged with these same tolerances.
PIN_TOL = {"m": dict(rtol=2.5e-7, atol=5e-11), "v": dict(rtol=3e-7, atol=1e-20),
           "theta": dict(rtol=1e-6, atol=2e-8)}


def torch_pin_ok(ours, theirs):
    """True if (theta, m, v) agree with torch's AdamW within the pin's tolerances."""
    return all(np.allclose(a, b, **PIN_TOL[k])
               for k, a, b in zip(("theta", "m", "v"), ours, theirs))


def _mutant(monkeypatch, kind):
    real = oa.adamw

    def mutated(theta, m, v, g, coef, lr, beta1, beta2, eps, weight_decay, step):
        f = np.float32
        gc = g * f(coef)
        m1 = f(beta1) * m + f(1 - beta1) * gc
        v1 = f(beta2) * v + f(1 - beta2) * gc * gc
        bc1, bc2 = f(1 - beta1 ** step), f(1 - beta2 ** step)
        if kind == "no_bias_correction":
            bc1 = bc2 = f(1)
        if kind == "eps_inside_sqrt":
            u = (m1 / bc1) / np.sqrt(v1 / bc2 + f(eps))
        else:
            u = (m1 / bc1) / (np.sqrt(v1 / bc2) + f(eps))
        if kind == "l2_not_decoupled":
            return real(theta, m, v, g + f(weight_decay) * theta, coef, lr, beta1, beta2, eps,
                        0.0, step)
        if kind == "bias_exponent_off_by_one":
            bc1, bc2 = f(1 - beta1 ** (step - 1)), f(1 - beta2 ** (step - 1))
            u = (m1 / bc1) / (np.sqrt(v1 / bc2) + f(eps))
        if kind == "no_clip":
            return real(theta, m, v, g, 1.0, lr, beta1, beta2, eps, weight_decay, step)
        if kind == "betas_swapped":
            m1 = f(beta2) * m + f(1 - beta2) * gc
            v1 = f(beta1) * v + f(1 - beta1) * gc * gc
            u = (m1 / bc1) / (np.sqrt(v1 / bc2) + f(eps))
        if kind == "decay_sign":
            th = theta * f(1 + lr * weight_decay) - f(lr) * u
        else:
            th = theta * f(1 - lr * weight_decay) - f(lr) * u
        return th, m1, v1, None
    return mutated


@pytest.mark.parametrize("kind", ["no_bias_correction", "eps_inside_sqrt", "l2_not_decoupled",
                                  "decay_sign", "bias_exponent_off_by_one", "no_clip",
                                  "betas_swapped"])
def test_planted_mistakes_fail_the_torch_pin(kind, monkeypatch):
    th, m, v, g = state(20000, seed=9)
    v = (v * np.float32(1e-4)).astype(np.float32)      # small v so eps matters
    c = np.float32(0.0345)
    bad = _mutant(monkeypatch, kind)(th, m, v, g, c, HP.lr, HP.beta1, HP.beta2, HP.eps,
                                     HP.weight_decay, HP.step)
    tth, tm, tv = torch_adamw(th, m, v, g, c)
    assert torch_pin_ok(run(th, m, v, g, c)[:3], (tth, tm, tv))    # the real update passes here
    assert not torch_pin_ok(bad[:3], (tth, tm, tv))


def test_bf16_output_is_rne_of_theta():
    th, m, v, g = state(4096)
    th1, _, _, p = run(th, m, v, g)
    want = torch.from_numpy(th1).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(p, want)
