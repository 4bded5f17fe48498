"""AdamW through the C ABI against the oracle: ragged sizes, clipping on and
off, several steps from the same seeded state, determinism, and the flat
adapter arena the stack trains."""
import numpy as np
import pytest
import torch

from layer_streamed_frozen_amd import binding as B
from layer_streamed_frozen_amd import store as S
from layer_streamed_frozen_amd import synth
from oracle import optim as O
from tests.test_gpu_layer import SMALL

pytestmark = pytest.mark.gpu


def _state(name, n):
    p = synth.normal(name + ".p", (n,), 0.05).astype(np.float32)
    z = np.zeros(n, np.float32)
    return p, z, z.copy()


def _grads(name, n, steps):
    return [synth.normal(f"{name}.g{t}", (n,), 2e-3).astype(np.float32) for t in range(steps)]


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def f32(x):
    """The value an fp32 field of the ABI's config holds."""
    return float(np.float32(x))


@pytest.mark.parametrize("n,clip,wd", [(1, 0.0, 0.0), (4099, 0.0, 0.01), (1_000_003, 0.05, 0.01),
                                       (3_145_728, 1.0, 0.0)])
def test_adamw_matches_oracle_over_steps(n, clip, wd):
    print(f"[adamw] n={n} clip={clip} wd={wd}", flush=True)
    steps, lr, b1, b2, eps = 4, 1e-3, 0.9, 0.999, 1e-8
    p0, m0, v0 = _state(f"adam{n}", n)
    gs = _grads(f"adam{n}", n, steps)
    p, m, v = _dev(p0), _dev(m0), _dev(v0)
    ws = torch.empty(B.adamw_workspace_bytes(), dtype=torch.uint8, device="cuda")
    norm = torch.zeros(1, dtype=torch.float32, device="cuda")
    cfg = B.AdamwCfg(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd, max_grad_norm=clip, step=0)
    op, om, ov = [p0.astype(np.float64)], [m0.astype(np.float64)], [v0.astype(np.float64)]
    for t in range(1, steps + 1):
        g = _dev(gs[t - 1])
        cfg.step = t
        B.adamw_step(p, g, m, v, cfg, norm, ws)
        torch.cuda.synchronize()
        # the oracle runs in fp64 on the hyper-parameters the fp32 config holds
        op, om, ov, onorm = O.adamw_step(op, [gs[t - 1]], om, ov, t, lr=f32(lr), beta1=f32(b1), beta2=f32(b2),
                                         eps=f32(eps), weight_decay=f32(wd), max_grad_norm=f32(clip))
        gn = float(norm.item())
        print(f"  t={t}: norm gpu={gn:.7e} oracle={onorm:.7e}", flush=True)
        assert abs(gn - onorm) <= 1e-5 * onorm
    # fp32 against fp64: each step rounds p once (half an ulp, 2^-24 |p|) and
    # computes the update to a few fp32 ulps of lr; the bound allows twice that
    pg, mg, vg = (x.double().cpu().numpy() for x in (p, m, v))
    dp = np.abs(pg - op[0])
    bound = steps * (2.0 ** -23 * np.maximum(np.abs(op[0]), np.abs(p0)) + 1e-6 * lr)
    print(f"  max|dp|={dp.max():.3e} worst dp/bound={float((dp / bound).max()):.3f} "
          f"max|dm|={np.abs(mg - om[0]).max():.3e} max|dv|={np.abs(vg - ov[0]).max():.3e}", flush=True)
    assert np.all(dp <= bound)
    np.testing.assert_allclose(mg, om[0], rtol=1e-5, atol=1e-6 * np.abs(om[0]).max())
    np.testing.assert_allclose(vg, ov[0], rtol=1e-5, atol=1e-6 * np.abs(ov[0]).max())


def test_adamw_deterministic_and_grad_untouched():
    n = 2_000_001
    p0, m0, v0 = _state("adet", n)
    g0 = _grads("adet", n, 1)[0]
    ws = torch.empty(B.adamw_workspace_bytes(), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        p, m, v, g = _dev(p0), _dev(m0), _dev(v0), _dev(g0)
        norm = torch.zeros(1, dtype=torch.float32, device="cuda")
        cfg = B.AdamwCfg(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, max_grad_norm=0.01, step=1)
        B.adamw_step(p, g, m, v, cfg, norm, ws)
        torch.cuda.synchronize()
        assert torch.equal(g, _dev(g0))
        outs.append((p, m, v, norm))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_adamw_bad_arguments():
    t = torch.zeros(8, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.adamw_workspace_bytes(), dtype=torch.uint8, device="cuda")
    for kw in (dict(step=0), dict(beta1=1.0), dict(eps=0.0), dict(lr=-1.0), dict(max_grad_norm=-1.0)):
        base = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, max_grad_norm=0.0, step=1)
        base.update(kw)
        with pytest.raises(B.LsfError) as e:
            B.adamw_step(t, t, t, t, B.AdamwCfg(**base), None, ws)
        assert e.value.status == B.LSF_ERR_INVALID_ARG
    with pytest.raises(B.LsfError) as e:
        B.adamw_step(t[1:], t, t, t, B.AdamwCfg(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, step=1), None, ws, n=4)
    assert e.value.status == B.LSF_ERR_ALIGN


def test_arena_update_equals_per_tensor_updates():
    lora = S.LoraSet(SMALL, 2, prefix="arena")
    for i in range(2):
        for n in lora.targets:
            lora.dA[i][n].copy_(torch.from_numpy(synth.normal(f"arena.g{i}{n}A", tuple(lora.dA[i][n].shape), 1e-3)))
            lora.dB[i][n].copy_(torch.from_numpy(synth.normal(f"arena.g{i}{n}B", tuple(lora.dB[i][n].shape), 1e-3)))
    before = {(i, n): (lora.A[i][n].clone(), lora.B[i][n].clone()) for i in range(2) for n in lora.targets}
    opt = S.AdamW(lora, lr=1e-3, weight_decay=0.01)
    opt.step()
    opt.step()
    torch.cuda.synchronize()
    ws = torch.empty(B.adamw_workspace_bytes(), dtype=torch.uint8, device="cuda")
    for (i, n), (a0, b0) in before.items():
        for p0, g, got in ((a0, lora.dA[i][n], lora.A[i][n]), (b0, lora.dB[i][n], lora.B[i][n])):
            p = p0.clone().reshape(-1)
            m, v = torch.zeros_like(p), torch.zeros_like(p)
            for t in (1, 2):
                cfg = B.AdamwCfg(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=t)
                B.adamw_step(p, g.reshape(-1).contiguous(), m, v, cfg, None, ws)
            torch.cuda.synchronize()
            assert torch.equal(p.view_as(got), got)
    # the zero padding between tensors stays zero
    used = sum(x.numel() for d in (lora.A, lora.B) for l in d for x in l.values())
    assert int((lora.params != 0).sum()) <= used
