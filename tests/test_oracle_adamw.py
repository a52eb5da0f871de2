"""Pins of the oracle's AdamW step (decoupled weight decay; the hotdry.top
Unsloth post, paged-optimizer section: Adam keeps a first and a second moment
per trainable parameter in 32-bit state).  The oracle is checked against
torch's own AdamW in float64 (a library implementation of the same published
rule) and against closed forms that a dropped bias correction, a coupled
decay or swapped betas would break."""
import numpy as np
import pytest
import torch

import oracle

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def _torch_adamw(p0, grads, lr, beta1, beta2, eps, weight_decay):
    p = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([p], lr=lr, betas=(beta1, beta2), eps=eps, weight_decay=weight_decay,
                            foreach=False, fused=False)
    for g in grads:
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("hp", [HP, dict(HP, weight_decay=0.0), dict(lr=3e-2, beta1=0.5, beta2=0.9, eps=1e-6,
                                                                    weight_decay=0.01)])
def test_adamw_matches_torch_float64(hp):
    rng = np.random.default_rng(7)
    p0 = rng.standard_normal(1000) * 0.02
    grads = [rng.standard_normal(1000) * s for s in (1.0, 1e-3, 5.0, 0.0, 1e-6)]
    tp, tm, tv = _torch_adamw(p0, grads, **hp)
    p, m, v = p0.copy(), np.zeros(1000), np.zeros(1000)
    for t, g in enumerate(grads, start=1):
        p, m, v = oracle.adamw_step(p, m, v, g, step=t, **hp)
    np.testing.assert_allclose(m, tm, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(v, tv, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(p, tp, rtol=1e-12, atol=1e-18)


def test_adamw_constant_gradient_closed_form():
    """g constant, no decay: m/(1-b1^t) = g and v/(1-b2^t) = g^2 exactly, so
    every step moves p by lr g / (|g| + eps)."""
    c = np.array([3.0, -0.25, 1e-5, -7.5])
    p = np.array([0.1, 0.2, -0.3, 0.0])
    p0 = p.copy()
    m = np.zeros(4)
    v = np.zeros(4)
    hp = dict(HP, weight_decay=0.0)
    for t in range(1, 6):
        p, m, v = oracle.adamw_step(p, m, v, c, step=t, **hp)
        want = p0 - t * hp["lr"] * c / (np.abs(c) + hp["eps"])
        np.testing.assert_allclose(p, want, rtol=1e-12, atol=1e-15)


def test_adamw_zero_gradient_is_pure_decay():
    """g = 0 leaves m = v = 0 and the update term 0, so p decays by (1 - lr wd)
    per step (decoupled decay, not folded into the gradient)."""
    p0 = np.array([1.0, -2.0, 0.5, 1e-30])
    p, m, v = p0.copy(), np.zeros(4), np.zeros(4)
    for t in range(1, 4):
        p, m, v = oracle.adamw_step(p, m, v, np.zeros(4), step=t, **HP)
    np.testing.assert_allclose(p, p0 * (1 - HP["lr"] * HP["weight_decay"]) ** 3, rtol=1e-14)
    assert not m.any() and not v.any()


def test_adamw_first_step_magnitude():
    """At t = 1 the bias-corrected step is lr g / (|g| + eps) whatever b1, b2
    are, for any single gradient (the step-one property of Adam)."""
    rng = np.random.default_rng(3)
    g = rng.standard_normal(64) * 10.0 ** rng.integers(-4, 3, 64)
    for b1, b2 in ((0.9, 0.999), (0.0, 0.5), (0.99, 0.9999)):
        p, m, v = oracle.adamw_step(np.zeros(64), np.zeros(64), np.zeros(64), g, lr=0.5, beta1=b1, beta2=b2,
                                    eps=1e-8, weight_decay=0.0, step=1)
        np.testing.assert_allclose(p, -0.5 * g / (np.abs(g) + 1e-8), rtol=1e-12)


def test_bf16_of_master_rounds_fp32():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, -2.5, 1e-40], dtype=np.float64)
    got = oracle.bf16_of_master(x)
    assert list(got[:4]) == [0x3F80, 0x3F80, 0x3F81, 0xC020]   # ties to even at 1 + 2^-8; 1 + 0.75 ulp rounds up
