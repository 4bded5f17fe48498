"""Pins for the DPO oracle."""
import numpy as np
import torch

from oracle import dpo as D
from oracle import model as M
from tests.test_oracle_model import _cfg, _fd_check, _sample, _weights


def test_sequence_logprobs_match_torch():
    rng = np.random.default_rng(30)
    B, T, V = 3, 7, 21
    z = rng.standard_normal((B * T, V)) * 2
    ids = rng.integers(0, V, (B, T))
    lp = D.sequence_logprobs(z, ids)
    ls = torch.log_softmax(torch.from_numpy(z), dim=1).numpy().reshape(B, T, V)
    ref = np.array([sum(ls[b, t, ids[b, t + 1]] for t in range(T - 1)) for b in range(B)])
    np.testing.assert_allclose(lp, ref, rtol=1e-12, atol=1e-12)


def test_identical_policy_and_reference_give_ln2():
    lp = np.array([-3.0, -5.5, -4.0, -1.0])
    loss, d = D.dpo_loss(lp, lp.copy(), 0.1)
    assert loss == np.log(2.0)
    np.testing.assert_allclose(d, [-0.025, -0.025, 0.025, 0.025])


def test_swapping_chosen_and_rejected():
    rng = np.random.default_rng(31)
    pi, ref = rng.standard_normal(4) * 3, rng.standard_normal(4) * 3
    l1, d1 = D.dpo_loss(pi, ref, 0.1)
    sw = np.r_[2, 3, 0, 1]
    l2, d2 = D.dpo_loss(pi[sw], ref[sw], 0.1)
    h = (pi[:2] - ref[:2]) - (pi[2:] - ref[2:])
    assert abs(l1 - np.mean(np.log1p(np.exp(-0.1 * h)))) < 1e-14
    assert abs(l2 - np.mean(np.log1p(np.exp(0.1 * h)))) < 1e-14
    np.testing.assert_allclose(d1.sum(), 0.0, atol=1e-15)


def test_dpo_step_finite_differences():
    cfg = _cfg()
    rng = np.random.default_rng(32)
    Ws, Ls = zip(*[_weights(cfg, rng) for _ in range(2)])
    Ws, Ls = list(Ws), list(Ls)
    V = 48
    ids = rng.integers(0, V, (4, 6))
    emb = rng.standard_normal((V, cfg.hidden))
    head = rng.standard_normal((V, cfg.hidden)) * 0.3
    fnorm = np.ones(cfg.hidden)

    def f():
        ref, _ = M.stack_forward(ids, emb, Ws, [None, None], fnorm, head, cfg, round_boundaries=False)
        pol, _ = M.stack_forward(ids, emb, Ws, Ls, fnorm, head, cfg, round_boundaries=False)
        return D.dpo_loss(D.sequence_logprobs(pol, ids), D.sequence_logprobs(ref, ids), 0.1)[0]

    out = D.dpo_step(ids, emb, Ws, Ls, fnorm, head, cfg, round_boundaries=False)
    assert abs(out["loss"] - f()) < 1e-12
    for i in range(2):
        for n in ("q", "v", "up"):
            A, Bm = Ls[i][n]
            dA, dB = out["grads"][i][n]
            _fd_check(f, A, dA, _sample(A.shape, rng, 3), rtol=5e-6, atol=1e-10)
            _fd_check(f, Bm, dB, _sample(Bm.shape, rng, 3), rtol=5e-6, atol=1e-10)


def test_zero_b_adapters_make_reference_equal_policy():
    cfg = _cfg()
    rng = np.random.default_rng(33)
    W, L = _weights(cfg, rng)
    L0 = {n: (A, np.zeros_like(B)) for n, (A, B) in L.items()}
    V = 32
    ids = rng.integers(0, V, (2, 5))
    emb = rng.standard_normal((V, cfg.hidden))
    head = rng.standard_normal((V, cfg.hidden)) * 0.3
    out = D.dpo_step(ids, emb, [W], [L0], np.ones(cfg.hidden), head, cfg)
    np.testing.assert_array_equal(out["lp_pi"], out["lp_ref"])
    assert out["loss"] == np.log(2.0)
