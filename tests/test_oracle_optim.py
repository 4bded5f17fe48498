"""Pins for the AdamW oracle."""
import numpy as np
import torch

from oracle import optim as O


def _tensors(rng, shapes, scale=1.0):
    return [rng.standard_normal(s) * scale for s in shapes]


def test_matches_torch_adamw_over_steps():
    rng = np.random.default_rng(40)
    shapes = [(8, 32), (48, 8), (5,)]
    p = _tensors(rng, shapes)
    tp = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in p]
    opt = torch.optim.AdamW(tp, lr=3e-3, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1)
    m = [np.zeros(s) for s in shapes]
    v = [np.zeros(s) for s in shapes]
    for t in range(1, 6):
        g = _tensors(rng, shapes, 0.5)
        for x, gg in zip(tp, g):
            x.grad = torch.tensor(gg)
        opt.step()
        p, m, v, _ = O.adamw_step(p, g, m, v, t, lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    for x, y in zip(p, tp):
        np.testing.assert_allclose(x, y.detach().numpy(), rtol=1e-13, atol=1e-15)
    st = opt.state[tp[0]]
    np.testing.assert_allclose(m[0], st["exp_avg"].numpy(), rtol=1e-13)
    np.testing.assert_allclose(v[0], st["exp_avg_sq"].numpy(), rtol=1e-13)


def test_clipping_matches_torch_clip_grad_norm():
    rng = np.random.default_rng(41)
    shapes = [(16, 16), (7, 3)]
    g = _tensors(rng, shapes, 2.0)
    tg = [torch.zeros(s, dtype=torch.float64, requires_grad=True) for s in shapes]
    for x, gg in zip(tg, g):
        x.grad = torch.tensor(gg)
    total = torch.nn.utils.clip_grad_norm_(tg, max_norm=1.5)
    assert abs(O.global_grad_norm(g) - float(total)) < 1e-12
    f = O.clip_factor(O.global_grad_norm(g), 1.5)
    for x, gg in zip(tg, g):
        np.testing.assert_allclose(gg * f, x.grad.numpy(), rtol=1e-14)
    # below the threshold nothing changes
    assert O.clip_factor(0.5, 1.5) == 1.0
    assert O.clip_factor(123.0, 0.0) == 1.0


def test_first_step_closed_form():
    # t = 1, no decay: m_hat = g, v_hat = g^2, so p moves by lr * g / (|g| + eps)
    rng = np.random.default_rng(42)
    p0 = rng.standard_normal(64)
    g = rng.standard_normal(64)
    z = np.zeros(64)
    (p1,), _, _, _ = O.adamw_step([p0], [g], [z], [z], 1, lr=1e-2, eps=1e-8)
    np.testing.assert_allclose(p0 - p1, 1e-2 * g / (np.abs(g) + 1e-8), rtol=1e-12)


def test_zero_gradient_only_decays():
    p0 = np.linspace(-1, 1, 9)
    z = np.zeros(9)
    (p1,), (m1,), (v1,), n = O.adamw_step([p0], [z], [z], [z], 3, lr=0.5, weight_decay=0.2)
    np.testing.assert_array_equal(m1, z)
    np.testing.assert_array_equal(v1, z)
    assert n == 0.0
    np.testing.assert_allclose(p1, p0 * (1 - 0.5 * 0.2), rtol=1e-15)
