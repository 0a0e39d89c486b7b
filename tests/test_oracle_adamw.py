"""Pins of the fp64 AdamW oracle (no GPU).

Each pin is fixed by the mathematics of the update, not by retyping it:
  * first step from zero moments: m^ = g and v^ = g^2 exactly, so the
    update is g / (|g| + eps), a sign-like step of size lr;
  * a constant gradient from zero moments keeps m^ = g and v^ = g^2 at every
    step, so the weight follows the geometric recursion
    W_t = c^t W_0 - lr u (1 - c^t) / (1 - c), c = 1 - lr wd, u = g / (|g| + eps);
  * a zero gradient from zero moments only decays the weight;
  * torch.optim.AdamW (a library implementation of Adam with decoupled
    weight decay), run in float64 on the CPU over several steps of random
    gradients, gives the same weights and moments.
Planted mistakes each of these catch: a missing bias correction (constant
gradient, torch), eps inside the square root (first step), decay applied
after the update or coupled into the gradient (torch), beta1/beta2 swapped
(torch), a wrong step exponent (constant gradient).
"""

import numpy as np
import pytest

import oracle


def test_first_step_closed_form():
    rng = np.random.default_rng(5)
    W = rng.standard_normal((7, 9))
    g = rng.standard_normal((7, 9)) * 1e-3
    lr, wd, eps = 0.01, 0.1, 1e-8
    Wn, m, v = oracle.adamw_step(W, g, np.zeros_like(W), np.zeros_like(W), step=1, lr=lr,
                                 weight_decay=wd, eps=eps)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v, 0.001 * g * g, rtol=1e-12)
    want = W * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    np.testing.assert_allclose(Wn, want, rtol=1e-13, atol=1e-16)


@pytest.mark.parametrize("steps", [1, 3, 25])
def test_constant_gradient_closed_form(steps):
    rng = np.random.default_rng(11 + steps)
    W0 = rng.standard_normal(50)
    g = rng.standard_normal(50)
    lr, wd, eps, b1, b2 = 0.003, 0.5, 1e-6, 0.8, 0.95
    W, m, v = W0, np.zeros(50), np.zeros(50)
    for t in range(1, steps + 1):
        W, m, v = oracle.adamw_step(W, g, m, v, step=t, lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd)
    c = 1 - lr * wd
    u = g / (np.abs(g) + eps)
    want = c ** steps * W0 - lr * u * (1 - c ** steps) / (1 - c)
    np.testing.assert_allclose(W, want, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(m, (1 - b1 ** steps) * g, rtol=1e-12)
    np.testing.assert_allclose(v, (1 - b2 ** steps) * g * g, rtol=1e-12)


def test_zero_gradient_only_decays():
    W = np.arange(12.0).reshape(3, 4) - 5.0
    Wn, m, v = oracle.adamw_step(W, np.zeros_like(W), np.zeros_like(W), np.zeros_like(W), step=4, lr=0.1,
                                 weight_decay=0.2)
    np.testing.assert_array_equal(Wn, W * (1 - 0.02))
    assert not m.any() and not v.any()


def test_matches_torch_adamw_float64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(23)
    shape = (13, 17)
    W0 = rng.standard_normal(shape)
    lr, b1, b2, eps, wd = 0.002, 0.85, 0.99, 1e-7, 0.3
    p = torch.nn.Parameter(torch.tensor(W0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    W, m, v = W0, np.zeros(shape), np.zeros(shape)
    for t in range(1, 8):
        g = rng.standard_normal(shape) * 10.0 ** rng.integers(-4, 1)
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        W, m, v = oracle.adamw_step(W, g, m, v, step=t, lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd)
        st = opt.state[p]
        np.testing.assert_allclose(W, p.detach().numpy(), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-300)


def test_rejects_step_zero():
    with pytest.raises(ValueError):
        oracle.adamw_step(np.zeros(2), np.zeros(2), np.zeros(2), np.zeros(2), step=0, lr=0.1)
