"""Pins for the layer / stack oracle.

Forward pieces are checked against library routines (torch CPU, fp64) or an
independent formulation; every backward is checked against fp64 central finite
differences on tiny shapes; plus the special cases the method has.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import model as M

TINY = dict(hidden=64, intermediate=96, n_heads=4, n_kv_heads=2, head_dim=16,
            rms_eps=1e-5, rope_theta=10000.0, lora_scale=1.5)


def _cfg(**kw):
    d = dict(TINY)
    d.update(kw)
    return M.LayerShape(**d)


def _weights(cfg, rng, rank=4, lora=True, std=0.2):
    W, L = {}, {}
    for n, (o, i) in cfg.proj_shapes().items():
        W[n] = rng.standard_normal((o, i)) * std
        L[n] = (rng.uniform(-0.3, 0.3, (rank, i)), rng.standard_normal((o, rank)) * 0.3) if lora else None
    W["norm1"] = 1.0 + 0.1 * rng.standard_normal(cfg.hidden)
    W["norm2"] = 1.0 + 0.1 * rng.standard_normal(cfg.hidden)
    return W, L


# ----------------------------------------------------------- library pins

def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 64))
    w = rng.standard_normal(64)
    y, _ = M.rmsnorm_fwd(x, w, 1e-5)
    ref = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(w), eps=1e-5).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    y1, _ = M.rmsnorm_fwd(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y1 ** 2, axis=1)), 1.0, rtol=1e-12)


def test_swiglu_matches_torch():
    rng = np.random.default_rng(1)
    g, u = rng.standard_normal((2, 50))
    ref = (F.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    np.testing.assert_allclose(M.swiglu_fwd(g, u), ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("nq,nkv", [(4, 2), (4, 4), (8, 1)])
def test_attention_matches_torch_sdpa(nq, nkv):
    rng = np.random.default_rng(2)
    T, d = 11, 16
    q = rng.standard_normal((T, nq, d))
    k = rng.standard_normal((T, nkv, d))
    v = rng.standard_normal((T, nkv, d))
    o, _ = M.attention_fwd(q, k, v)
    tq, tk, tv = (torch.from_numpy(a).permute(1, 0, 2)[None] for a in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_attention_single_token_returns_value():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 8, 16))
    k = rng.standard_normal((1, 2, 16))
    v = rng.standard_normal((1, 2, 16))
    o, _ = M.attention_fwd(q, k, v)
    for h in range(8):
        np.testing.assert_array_equal(o[0, h], v[0, h // 4])


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(4)
    T, nh, d = 9, 3, 16
    x = rng.standard_normal((T, nh, d))
    ang = M.rope_angles(T, d, 10000.0)
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * ang)[:, None, :]
    ref = np.concatenate([z.real, z.imag], axis=-1)
    np.testing.assert_allclose(M.rope_fwd(x, ang), ref, rtol=1e-12, atol=1e-12)
    # position 0 is the identity, pair norms are preserved
    np.testing.assert_array_equal(M.rope_fwd(x, ang)[0], x[0])
    y = M.rope_fwd(x, ang)
    np.testing.assert_allclose(y[..., :8] ** 2 + y[..., 8:] ** 2, x[..., :8] ** 2 + x[..., 8:] ** 2,
                               rtol=1e-12)
    # inv_freq = theta^(-2i/d): i = 1 at position 1 gives 10000^(-1/8)
    assert abs(ang[1, 1] - 10000.0 ** (-2.0 / 16)) < 1e-15


def test_cross_entropy_matches_torch():
    rng = np.random.default_rng(5)
    z = rng.standard_normal((12, 33)) * 3
    labels = rng.integers(0, 33, 12)
    valid = np.ones(12, bool)
    valid[[3, 11]] = False
    loss, dz = M.cross_entropy_fwd_bwd(z, labels, valid)
    tz = torch.from_numpy(z).requires_grad_(True)
    ref = F.cross_entropy(tz[torch.from_numpy(valid)], torch.from_numpy(labels[valid]))
    ref.backward()
    assert abs(loss - ref.item()) < 1e-12
    np.testing.assert_allclose(dz, tz.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(dz.sum(axis=1), 0.0, atol=1e-15)


def test_zero_head_gives_log_vocab():
    cfg = _cfg()
    rng = np.random.default_rng(6)
    W, L = _weights(cfg, rng)
    V = 40
    ids = rng.integers(0, V, (2, 6))
    emb = rng.standard_normal((V, cfg.hidden))
    out = M.stack_step(ids, emb, [W], [L], np.ones(cfg.hidden), np.zeros((V, cfg.hidden)), cfg)
    assert abs(out["loss"] - np.log(V)) < 1e-12


# ----------------------------------------------------------- invariants

def test_lora_b_zero_reproduces_base():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 32))
    W = rng.standard_normal((24, 32))
    A = rng.standard_normal((4, 32))
    y, _ = M.lora_linear_fwd(x, W, A, np.zeros((24, 4)), 2.0)
    np.testing.assert_array_equal(y, x @ W.T)
    dy = rng.standard_normal((5, 24))
    dx, dA, dB = M.lora_linear_bwd(dy, x, W, A, np.zeros((24, 4)), 2.0, x @ A.T)
    np.testing.assert_array_equal(dA, 0.0)
    assert np.any(dB != 0)


def test_layer_with_zero_b_equals_adapterless_layer():
    cfg = _cfg()
    rng = np.random.default_rng(8)
    W, L = _weights(cfg, rng)
    L0 = {n: (A, np.zeros_like(B)) for n, (A, B) in L.items()}
    x = rng.standard_normal((2, 6, cfg.hidden))
    y0, _ = M.layer_fwd(x, W, L0, cfg)
    y1, _ = M.layer_fwd(x, W, None, cfg)
    np.testing.assert_array_equal(y0, y1)


def test_layer_is_causal():
    cfg = _cfg()
    rng = np.random.default_rng(9)
    W, L = _weights(cfg, rng)
    x = rng.standard_normal((1, 8, cfg.hidden))
    y, _ = M.layer_fwd(x, W, L, cfg)
    x2 = x.copy()
    x2[0, 5] += rng.standard_normal(cfg.hidden)
    y2, _ = M.layer_fwd(x2, W, L, cfg)
    np.testing.assert_array_equal(y[0, :5], y2[0, :5])
    assert np.any(y[0, 5] != y2[0, 5])


def test_mha_special_case_matches_torch_layer_pieces():
    # nkv == nq: grouped attention reduces to plain multi-head attention
    rng = np.random.default_rng(10)
    q, k, v = rng.standard_normal((3, 6, 4, 8))
    o, _ = M.attention_fwd(q, k, v)
    tq, tk, tv = (torch.from_numpy(a).permute(1, 0, 2)[None] for a in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


# ------------------------------------------------------ finite differences

def _fd_check(f, param, analytic, idxs, eps=1e-6, rtol=2e-6, atol=1e-9):
    for ix in idxs:
        old = param[ix]
        param[ix] = old + eps
        fp = f()
        param[ix] = old - eps
        fm = f()
        param[ix] = old
        num = (fp - fm) / (2 * eps)
        assert abs(num - analytic[ix]) <= atol + rtol * max(abs(num), abs(analytic[ix])), \
            (ix, num, analytic[ix])


def _sample(shape, rng, n=6):
    return [tuple(int(rng.integers(0, s)) for s in shape) for _ in range(n)]


def test_lora_linear_finite_differences():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 12))
    W = rng.standard_normal((9, 12))
    A = rng.standard_normal((3, 12))
    B = rng.standard_normal((9, 3))
    R = rng.standard_normal((5, 9))
    s = 2.0

    def f():
        return float(np.sum(M.lora_linear_fwd(x, W, A, B, s)[0] * R))

    _, u = M.lora_linear_fwd(x, W, A, B, s)
    dx, dA, dB = M.lora_linear_bwd(R, x, W, A, B, s, u)
    # closed forms: dB = s dY^T (X A^T), dA = s (dY B)^T X
    np.testing.assert_allclose(dB, s * R.T @ (x @ A.T), rtol=1e-13)
    np.testing.assert_allclose(dA, (s * R @ B).T @ x, rtol=1e-13)
    for p, g in ((x, dx), (A, dA), (B, dB)):
        _fd_check(f, p, g, _sample(p.shape, rng))


def test_layer_finite_differences():
    cfg = _cfg()
    rng = np.random.default_rng(12)
    W, L = _weights(cfg, rng)
    x = rng.standard_normal((2, 8, cfg.hidden))
    R = rng.standard_normal((2, 8, cfg.hidden))

    def f():
        return float(np.sum(M.layer_fwd(x, W, L, cfg)[0] * R))

    _, cache = M.layer_fwd(x, W, L, cfg)
    dx, grads = M.layer_bwd(R, W, L, cfg, cache)
    assert set(grads) == set(M.PROJ)
    _fd_check(f, x, dx, _sample(x.shape, rng, 10))
    for n in M.PROJ:
        A, B = L[n]
        dA, dB = grads[n]
        _fd_check(f, A, dA, _sample(A.shape, rng, 4))
        _fd_check(f, B, dB, _sample(B.shape, rng, 4))


def test_layer_finite_differences_partial_adapters():
    # adapters on q and v only (the pages' narrow 8B setting)
    cfg = _cfg(n_kv_heads=4)
    rng = np.random.default_rng(13)
    W, L = _weights(cfg, rng)
    L = {n: (L[n] if n in ("q", "v") else None) for n in M.PROJ}
    x = rng.standard_normal((1, 7, cfg.hidden))
    R = rng.standard_normal((1, 7, cfg.hidden))

    def f():
        return float(np.sum(M.layer_fwd(x, W, L, cfg)[0] * R))

    _, cache = M.layer_fwd(x, W, L, cfg)
    dx, grads = M.layer_bwd(R, W, L, cfg, cache)
    assert set(grads) == {"q", "v"}
    _fd_check(f, x, dx, _sample(x.shape, rng, 8))
    for n in ("q", "v"):
        _fd_check(f, L[n][0], grads[n][0], _sample(L[n][0].shape, rng, 4))


def test_stack_finite_differences():
    cfg = _cfg()
    rng = np.random.default_rng(14)
    nL, V = 2, 64
    Ws, Ls = zip(*[_weights(cfg, rng) for _ in range(nL)])
    Ws, Ls = list(Ws), list(Ls)
    ids = rng.integers(0, V, (2, 6))
    emb = rng.standard_normal((V, cfg.hidden))
    head = rng.standard_normal((V, cfg.hidden)) * 0.1
    fnorm = 1.0 + 0.1 * rng.standard_normal(cfg.hidden)

    def f():
        logits, _ = M.stack_forward(ids, emb, Ws, Ls, fnorm, head, cfg, round_boundaries=False)
        lab, val = M.shifted_labels(ids)
        return M.cross_entropy_fwd_bwd(logits, lab, val)[0]

    out = M.stack_step(ids, emb, Ws, Ls, fnorm, head, cfg, round_boundaries=False)
    assert abs(out["loss"] - f()) < 1e-12
    np.testing.assert_allclose(out["dlogits"].sum(axis=1), 0.0, atol=1e-14)
    for i in range(nL):
        for n in ("q", "o", "down"):
            A, B = Ls[i][n]
            dA, dB = out["grads"][i][n]
            _fd_check(f, A, dA, _sample(A.shape, rng, 3))
            _fd_check(f, B, dB, _sample(B.shape, rng, 3))


def test_loss_scale_scales_gradients_only():
    cfg = _cfg()
    rng = np.random.default_rng(15)
    W, L = _weights(cfg, rng)
    V = 32
    ids = rng.integers(0, V, (1, 5))
    emb = rng.standard_normal((V, cfg.hidden))
    head = rng.standard_normal((V, cfg.hidden)) * 0.1
    a = M.stack_step(ids, emb, [W], [L], np.ones(cfg.hidden), head, cfg)
    b = M.stack_step(ids, emb, [W], [L], np.ones(cfg.hidden), head, cfg, loss_scale=0.25)
    assert a["loss"] == b["loss"]
    np.testing.assert_allclose(b["grads"][0]["up"][0], 0.25 * a["grads"][0]["up"][0], rtol=1e-12)


# --------------------------------------------------- bf16 rounding, batches

def test_round_bf16_matches_torch_cast():
    """The layer-boundary rounding the stack oracle applies (the checkpoints
    are bf16) is round-to-nearest-even: torch's bf16 cast on 10^5 values over
    the whole fp32 range (normals, subnormals, signed zeros) and hand-built
    ties.  A truncating rounding or a ties-away rule fails here."""
    from oracle import nf4 as onf4
    rng = np.random.default_rng(31)
    bits = rng.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32)
    bits = bits[((bits >> 23) & 0xFF) != 0xFF]  # finite values only
    x = np.concatenate([bits.view(np.float32),
                        rng.standard_normal(20000).astype(np.float32),
                        np.array([0.0, -0.0, 1e-45, -1e-45, 3.3895314e38], np.float32)])
    got = M.round_bf16(x)
    assert got.dtype == np.float32
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    # the same bits as the NF4 module's own rounding (two independent writings)
    np.testing.assert_array_equal(got.view(np.uint32) >> 16, onf4.bf16_round(x).astype(np.uint32))
    # exact ties go to the even neighbour; one ulp above a tie rounds up
    e = 2.0 ** -8  # half a bf16 ulp at 1.0
    cases = [(1 + e, 0x3F80), (1 + 3 * e, 0x3F82), (-(1 + e), 0xBF80), (1 + e + 2 ** -23, 0x3F81),
             (2 - e, 0x4000), (1 - e / 2, 0x3F80)]
    for v, want in cases:
        r = M.round_bf16(np.array([v], np.float32))
        assert int(r.view(np.uint32)[0]) >> 16 == want, (v, hex(int(r.view(np.uint32)[0])))
    # fp64 inputs are rounded through fp32, exactly as torch casts them
    x64 = rng.standard_normal(5000) * 3.0
    x64[:3] = [1 + e + 2 ** -40, -(1 + e + 2 ** -40), 1 + e]
    ref64 = torch.from_numpy(x64).to(torch.bfloat16).to(torch.float64).numpy()
    got64 = M.round_bf16(x64)
    assert got64.dtype == np.float64
    np.testing.assert_array_equal(got64, ref64)


def test_batched_layer_equals_per_sequence_calls():
    """A batch of sequences is a batch of independent sequences: RoPE
    positions restart at 0 and no query attends to another sequence.  The
    layer on a 3-sequence batch must equal three 1-sequence calls (output and
    input gradient per sequence; adapter gradients as their sum), and so must
    the rotated queries and keys it keeps.  Not bit for
    bit: BLAS blocks a [3T, H] product differently from a [T, H] one, which
    moves fp64 results by ~1e-14; a leaked position or cross-sequence
    attention moves them by O(1)."""
    cfg = _cfg()
    rng = np.random.default_rng(32)
    W, L = _weights(cfg, rng)
    nb, T = 3, 9
    x = rng.standard_normal((nb, T, cfg.hidden))
    dy = rng.standard_normal((nb, T, cfg.hidden))
    y, cache = M.layer_fwd(x, W, L, cfg)
    dx, grads = M.layer_bwd(dy, W, L, cfg, cache)
    gsum = {n: [np.zeros_like(a) for a in grads[n]] for n in grads}
    for b in range(nb):
        yb, cb = M.layer_fwd(x[b:b + 1], W, L, cfg)
        dxb, gb = M.layer_bwd(dy[b:b + 1], W, L, cfg, cb)
        # the rotated q and k themselves (attention scores depend only on
        # position differences, so the outputs alone cannot show an offset)
        np.testing.assert_allclose(cache["qr"][b], cb["qr"][0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(cache["kr"][b], cb["kr"][0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(y[b], yb[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dx[b], dxb[0], rtol=1e-12, atol=1e-12)
        for n in gb:
            for k in range(2):
                gsum[n][k] += gb[n][k]
    for n in grads:
        for k in range(2):
            np.testing.assert_allclose(grads[n][k], gsum[n][k], rtol=1e-11, atol=1e-12)
    # the same holds for the whole stack step: two sequences = two steps,
    # each with half the weight of the mean over labelled positions
    V = 48
    ids = rng.integers(0, V, (2, 7))
    emb = rng.standard_normal((V, cfg.hidden))
    head = rng.standard_normal((V, cfg.hidden)) * 0.1
    fn = np.ones(cfg.hidden)
    both = M.stack_step(ids, emb, [W], [L], fn, head, cfg)
    parts = [M.stack_step(ids[b:b + 1], emb, [W], [L], fn, head, cfg, loss_scale=0.5) for b in range(2)]
    np.testing.assert_allclose(both["logits"], np.concatenate([p["logits"] for p in parts]), rtol=1e-12,
                               atol=1e-12)
    assert abs(both["loss"] - 0.5 * (parts[0]["loss"] + parts[1]["loss"])) < 1e-12
    for n in M.PROJ:
        for k in range(2):
            np.testing.assert_allclose(both["grads"][0][n][k],
                                       parts[0]["grads"][0][n][k] + parts[1]["grads"][0][n][k],
                                       rtol=1e-10, atol=1e-13)
