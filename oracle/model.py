"""Oracle: LoRA linear, Llama-style decoder layer and streamed-stack step.

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

Everything here is the plain, un-streamed, un-checkpointed definition, in the
arrays' floating type (fp64 unless a caller asks otherwise), with hand-derived
backward formulas.  Sources, by page (the pages print no formulas; the
readings below are the plainest ones their text supports):

* Frozen base, trainable LoRA A/B only, adapters/gradients resident:
  news article "aizxs.com/ai-learning/13312.html", section on exact layer
  streaming; tutorial "alphalab.site/soup-layer-streaming", opening summary.
* The input gradient still needs the frozen weight, dL/dx = W^T dL/dy, and
  each layer's forward is recomputed in the backward walk: tutorial, section
  "four-stage data path", item 3, and FAQ 4.
* Resident untied embedding and lm_head, SFT cross-entropy: tutorial, section
  on why plain QLoRA can still miss 4 GB (the peak-memory breakdown) and the
  YAML of step 2 (task sft, r 16, alpha 16, dropout 0).
* Llama conventions (the tool loads HF causal-LM models; tutorial, "Step 2"
  YAML and "backend: transformers"): RMSNorm with the weight applied after
  normalising; rotate-half RoPE with inv_freq = theta^(-2i/d) and positions
  restarting at 0 in every sequence; grouped-query attention where query head
  h reads kv head h // (n_heads / n_kv_heads), scale 1/sqrt(d), causal mask
  including the diagonal; SwiGLU MLP a = silu(gate) * up.
* LoRA: y = x W^T + s (x A^T) B^T, s = alpha / r, dropout 0.

Backward formulas (dy is the incoming gradient):
  linear     dx = dy W + s (dy B) A;  dA = s (dy B)^T x;  dB = s dy^T (x A^T)
  rmsnorm    y = w * x * r, r = (mean x^2 + eps)^-1/2
             dx = r (w dy) - x r^3 sum_j (w dy)_j x_j / H
  rope       the transpose of a rotation: rotate dy by -angle
  attention  dV = P^T dO; dP = dO V^T; dS = P (dP - rowsum(dP P));
             dQ = dS K / sqrt(d); dK = dS^T Q / sqrt(d); GQA sums dK, dV
             over the query heads of a group
  swiglu     dg = da u s(g) (1 + g (1 - s(g))); du = da g s(g)
  CE         loss = mean over labelled positions of (lse(z) - z[label]);
             dz = (softmax(z) - onehot(label)) / count

Parity: forward pinned by library routines (torch CPU scaled-dot-product
attention, rms_norm, cross_entropy, silu; complex-number RoPE) and special
cases; backward pinned by fp64 central finite differences on tiny shapes;
``round_bf16`` pinned against torch's bf16 cast (random bit patterns and
hand-built ties); a batch pinned to equal its sequences run one at a time
(layer output, rotated q and k, input gradient, summed adapter gradients).
"""
import numpy as np

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


class LayerShape:
    """Shape and constants of one decoder layer."""

    def __init__(self, hidden, intermediate, n_heads, n_kv_heads, head_dim,
                 rms_eps=1e-5, rope_theta=500000.0, lora_scale=1.0):
        self.hidden = hidden
        self.intermediate = intermediate
        self.n_heads = n_heads
        self.n_kv_heads = n_kv_heads
        self.head_dim = head_dim
        self.rms_eps = rms_eps
        self.rope_theta = rope_theta
        self.lora_scale = lora_scale

    def proj_shapes(self):
        """[out, in] of every projection, in ``PROJ`` order."""
        H, I = self.hidden, self.intermediate
        q = self.n_heads * self.head_dim
        kv = self.n_kv_heads * self.head_dim
        return {"q": (q, H), "k": (kv, H), "v": (kv, H), "o": (H, q),
                "gate": (I, H), "up": (I, H), "down": (H, I)}


def round_bf16(x):
    """Round to the nearest bfloat16 (ties to even) via fp32; keep the dtype."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(x.dtype)


# ----------------------------------------------------------------- LoRA linear

def lora_linear_fwd(x, W, A, B, s):
    """y = x W^T + s (x A^T) B^T.  Returns (y, u = x A^T or None)."""
    y = x @ W.T
    u = None
    if A is not None:
        u = x @ A.T
        y = y + s * (u @ B.T)
    return y, u


def lora_linear_bwd(dy, x, W, A, B, s, u):
    """Returns (dx, dA, dB); dA and dB are None without an adapter."""
    dx = dy @ W
    if A is None:
        return dx, None, None
    du = s * (dy @ B)
    dx = dx + du @ A
    dA = du.T @ x
    dB = s * (dy.T @ u)
    return dx, dA, dB


# ---------------------------------------------------------------- elementwise

def rmsnorm_fwd(x, w, eps):
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * w, r


def rmsnorm_bwd(dy, x, w, r):
    g = dy * w
    dot = np.sum(g * x, axis=-1, keepdims=True)
    return r * g - x * (r ** 3) * dot / x.shape[-1]


def rope_angles(seq, head_dim, theta, dtype=np.float64):
    """angle[t, i] = t * theta^(-2i/d) for positions 0..seq-1."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    return np.outer(np.arange(seq, dtype=np.float64), inv_freq).astype(dtype)


def rope_fwd(x, ang):
    """Rotate-half RoPE.  x [T, heads, d], ang [T, d/2]."""
    h = x.shape[-1] // 2
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_bwd(dy, ang):
    h = dy.shape[-1] // 2
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    d1, d2 = dy[..., :h], dy[..., h:]
    return np.concatenate([d1 * c + d2 * s, d2 * c - d1 * s], axis=-1)


def swiglu_fwd(g, u):
    sg = 1.0 / (1.0 + np.exp(-g))
    return g * sg * u


def swiglu_bwd(da, g, u):
    sg = 1.0 / (1.0 + np.exp(-g))
    dg = da * u * sg * (1.0 + g * (1.0 - sg))
    du = da * g * sg
    return dg, du


# ------------------------------------------------------------------ attention

def attention_fwd(q, k, v):
    """Causal GQA for one sequence.  q [T, nq, d]; k, v [T, nkv, d].

    Returns (o [T, nq, d], P [nq, T, T] softmax probabilities).
    """
    T, nq, d = q.shape
    grp = nq // k.shape[1]
    scale = 1.0 / np.sqrt(d)
    future = np.triu(np.ones((T, T), dtype=bool), 1)
    o = np.empty_like(q)
    P = np.empty((nq, T, T), dtype=q.dtype)
    for h in range(nq):
        kv = h // grp
        s = (q[:, h, :] @ k[:, kv, :].T) * scale
        s[future] = -np.inf
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        P[h] = p
        o[:, h, :] = p @ v[:, kv, :]
    return o, P


def attention_bwd(do, q, k, v, P):
    T, nq, d = q.shape
    grp = nq // k.shape[1]
    scale = 1.0 / np.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(nq):
        kv = h // grp
        p = P[h]
        dv[:, kv, :] += p.T @ do[:, h, :]
        dp = do[:, h, :] @ v[:, kv, :].T
        ds = p * (dp - np.sum(dp * p, axis=1, keepdims=True))
        dq[:, h, :] = (ds @ k[:, kv, :]) * scale
        dk[:, kv, :] += (ds.T @ q[:, h, :]) * scale
    return dq, dk, dv


# -------------------------------------------------------------- decoder layer

def _lora(lora, name):
    if lora is None or lora.get(name) is None:
        return None, None
    return lora[name]


def layer_fwd(x, W, lora, cfg):
    """One decoder layer.

    x [B, T, H]; W dict of dense frozen weights ("q".."down" as [out, in],
    "norm1", "norm2" as [H]); lora dict name -> (A [r, in], B [out, r]) or
    None (no adapter / adapters disabled).  Returns (y, cache).
    """
    Bsz, T, H = x.shape
    nq, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    s = cfg.lora_scale
    ang = rope_angles(T, d, cfg.rope_theta, x.dtype)
    xf = x.reshape(Bsz * T, H)
    h1, r1 = rmsnorm_fwd(xf, W["norm1"], cfg.rms_eps)
    outs, us = {}, {}
    for n in ("q", "k", "v"):
        A, Bm = _lora(lora, n)
        outs[n], us[n] = lora_linear_fwd(h1, W[n], A, Bm, s)
    q = outs["q"].reshape(Bsz, T, nq, d)
    k = outs["k"].reshape(Bsz, T, nkv, d)
    v = outs["v"].reshape(Bsz, T, nkv, d)
    qr = np.empty_like(q)
    kr = np.empty_like(k)
    o = np.empty_like(q)
    Ps = []
    for b in range(Bsz):
        qr[b] = rope_fwd(q[b], ang)
        kr[b] = rope_fwd(k[b], ang)
        o[b], P = attention_fwd(qr[b], kr[b], v[b])
        Ps.append(P)
    of = o.reshape(Bsz * T, nq * d)
    A, Bm = _lora(lora, "o")
    ao, us["o"] = lora_linear_fwd(of, W["o"], A, Bm, s)
    x2 = xf + ao
    h2, r2 = rmsnorm_fwd(x2, W["norm2"], cfg.rms_eps)
    A, Bm = _lora(lora, "gate")
    g, us["gate"] = lora_linear_fwd(h2, W["gate"], A, Bm, s)
    A, Bm = _lora(lora, "up")
    u, us["up"] = lora_linear_fwd(h2, W["up"], A, Bm, s)
    a = swiglu_fwd(g, u)
    A, Bm = _lora(lora, "down")
    md, us["down"] = lora_linear_fwd(a, W["down"], A, Bm, s)
    y = x2 + md
    cache = dict(xf=xf, h1=h1, r1=r1, qr=qr, kr=kr, v=v, Ps=Ps, of=of, x2=x2,
                 h2=h2, r2=r2, g=g, u=u, a=a, us=us, ang=ang)
    return y.reshape(Bsz, T, H), cache


def layer_bwd(dy, W, lora, cfg, cache):
    """Backward of ``layer_fwd``.  Returns (dx [B, T, H], grads) where grads
    maps name -> (dA, dB) for every projection that has an adapter."""
    Bsz, T, H = dy.shape
    nq, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    s = cfg.lora_scale
    c = cache
    grads = {}
    dyf = dy.reshape(Bsz * T, H)

    def lin_bwd(name, dout, xin):
        A, Bm = _lora(lora, name)
        dx, dA, dB = lora_linear_bwd(dout, xin, W[name], A, Bm, s, c["us"][name])
        if dA is not None:
            grads[name] = (dA, dB)
        return dx

    da = lin_bwd("down", dyf, c["a"])
    dg, du = swiglu_bwd(da, c["g"], c["u"])
    dh2 = lin_bwd("gate", dg, c["h2"]) + lin_bwd("up", du, c["h2"])
    dx2 = dyf + rmsnorm_bwd(dh2, c["x2"], W["norm2"], c["r2"])
    dof = lin_bwd("o", dx2, c["of"])
    do = dof.reshape(Bsz, T, nq, d)
    dq = np.empty((Bsz, T, nq, d), dtype=dy.dtype)
    dk = np.empty((Bsz, T, nkv, d), dtype=dy.dtype)
    dv = np.empty((Bsz, T, nkv, d), dtype=dy.dtype)
    for b in range(Bsz):
        dqr, dkr, dv[b] = attention_bwd(do[b], c["qr"][b], c["kr"][b], c["v"][b], c["Ps"][b])
        dq[b] = rope_bwd(dqr, c["ang"])
        dk[b] = rope_bwd(dkr, c["ang"])
    dh1 = (lin_bwd("q", dq.reshape(Bsz * T, nq * d), c["h1"])
           + lin_bwd("k", dk.reshape(Bsz * T, nkv * d), c["h1"])
           + lin_bwd("v", dv.reshape(Bsz * T, nkv * d), c["h1"]))
    dx = dx2 + rmsnorm_bwd(dh1, c["xf"], W["norm1"], c["r1"])
    return dx.reshape(Bsz, T, H), grads


# ------------------------------------------------------------ head and stack

def cross_entropy_fwd_bwd(logits, labels, valid):
    """Mean CE over the positions where ``valid`` is true.

    logits [N, V]; labels [N] int; valid [N] bool.  Returns (loss, dlogits).
    """
    z = logits
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    ssum = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(ssum))[:, 0]
    idx = np.arange(z.shape[0])
    count = int(np.count_nonzero(valid))
    per = lse - z[idx, labels]
    loss = float(np.sum(per[valid]) / count)
    dz = e / ssum
    dz[idx, labels] -= 1.0
    dz[~valid] = 0.0
    return loss, dz / count


def shifted_labels(ids):
    """Next-token labels for ids [B, T]: position t predicts ids[t+1]; the last
    position of every sequence has no label."""
    Bsz, T = ids.shape
    labels = np.zeros((Bsz, T), dtype=np.int64)
    labels[:, :-1] = ids[:, 1:]
    valid = np.zeros((Bsz, T), dtype=bool)
    valid[:, :-1] = True
    return labels.reshape(-1), valid.reshape(-1)


def stack_forward(ids, emb, layers, loras, final_norm, head, cfg,
                  dtype=np.float64, round_boundaries=True, keep_caches=True):
    """Forward of the whole stack.

    ids [B, T] int; emb, head [V, H]; layers: indexable, layers[i] -> dense
    weight dict of layer i (may build it lazily); loras[i] -> LoRA dict or
    None.  With ``round_boundaries`` every layer output is rounded to bf16,
    the activation type the layer-to-layer checkpoints are stored in.
    Returns (logits [B*T, V], state for ``stack_backward``).
    """
    x = np.asarray(emb)[ids].astype(dtype)
    caches = []
    for i in range(len(loras)):
        y, cache = layer_fwd(x, layers[i], loras[i], cfg)
        caches.append(cache if keep_caches else None)
        x = round_bf16(y) if round_boundaries else y
    Bsz, T, H = x.shape
    xf = x.reshape(Bsz * T, H)
    hN, rN = rmsnorm_fwd(xf, np.asarray(final_norm, dtype=dtype), cfg.rms_eps)
    logits = hN @ np.asarray(head, dtype=dtype).T
    return logits, dict(caches=caches, xN=xf, hN=hN, rN=rN, shape=x.shape)


def stack_backward(dlogits, layers, loras, final_norm, head, cfg, state,
                   dtype=np.float64):
    """Backward of ``stack_forward`` given dL/dlogits.  Returns
    (per-layer list of LoRA grads dicts, dL/dx0)."""
    Bsz, T, H = state["shape"]
    dhN = dlogits @ np.asarray(head, dtype=dtype)
    dxf = rmsnorm_bwd(dhN, state["xN"], np.asarray(final_norm, dtype=dtype), state["rN"])
    dx = dxf.reshape(Bsz, T, H)
    grads = [None] * len(loras)
    for i in reversed(range(len(loras))):
        dx, grads[i] = layer_bwd(dx, layers[i], loras[i], cfg, state["caches"][i])
    return grads, dx


def stack_step(ids, emb, layers, loras, final_norm, head, cfg,
               dtype=np.float64, round_boundaries=True, loss_scale=1.0):
    """One SFT micro-batch: forward, CE over shifted labels, full backward.

    Returns dict(loss, logits, dlogits, grads) with grads[i][name] = (dA, dB),
    the gradient of loss_scale * loss.
    """
    logits, state = stack_forward(ids, emb, layers, loras, final_norm, head, cfg,
                                  dtype, round_boundaries)
    labels, valid = shifted_labels(ids)
    loss, dlogits = cross_entropy_fwd_bwd(logits, labels, valid)
    dlogits = dlogits * loss_scale
    grads, _ = stack_backward(dlogits, layers, loras, final_norm, head, cfg, state, dtype)
    return dict(loss=loss, logits=logits, dlogits=dlogits, grads=grads)
