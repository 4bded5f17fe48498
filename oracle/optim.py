"""Oracle: AdamW on the trainable adapter parameters, with optional clipping
of the global gradient norm.

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

Source: the tutorial page (alphalab.site/soup-layer-streaming, section "step 2:
one YAML") trains the adapters with an Adam-family optimizer with decoupled
weight decay ("paged_adamw_8bit") at lr 2e-4; the news page (section on what
the method can do) keeps the LoRA weights, their gradients and the optimizer
state on the GPU.  The pages give no formula, so the plain AdamW definition
(Loshchilov and Hutter, decoupled weight decay) is used, with fp32 state; the
pages' 8-bit paged state is not modelled.  For step t >= 1:

  g    <- g * min(1, c / (||g||_2 + 1e-6))     if a clip norm c > 0 is given,
                                               ||g|| over every tensor together
  p    <- p - lr * wd * p
  m    <- b1 m + (1 - b1) g
  v    <- b2 v + (1 - b2) g^2
  p    <- p - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)

Parity: pinned (torch.optim.AdamW over several steps, torch's
clip_grad_norm_ for the clipping factor, the closed form of the first step,
a zero gradient leaving only the decay).
"""
import numpy as np


def global_grad_norm(grads):
    """L2 norm over every gradient array together."""
    return float(np.sqrt(sum(float(np.sum(np.asarray(g, np.float64) ** 2)) for g in grads)))


def clip_factor(norm, max_norm):
    """Factor the gradients are multiplied by (1 when clipping is off)."""
    if max_norm <= 0:
        return 1.0
    return min(1.0, max_norm / (norm + 1e-6))


def adamw_step(params, grads, m, v, t, lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
               max_grad_norm=0.0):
    """One update of every (param, grad, m, v) quadruple, in fp64.  Returns
    (new params, new m, new v, gradient norm before clipping)."""
    norm = global_grad_norm(grads)
    f = clip_factor(norm, max_grad_norm)
    bc1 = 1.0 - beta1 ** t
    bc2 = 1.0 - beta2 ** t
    out_p, out_m, out_v = [], [], []
    for p, g, m0, v0 in zip(params, grads, m, v):
        p = np.asarray(p, np.float64)
        g = np.asarray(g, np.float64) * f
        p = p - lr * weight_decay * p
        m1 = beta1 * np.asarray(m0, np.float64) + (1.0 - beta1) * g
        v1 = beta2 * np.asarray(v0, np.float64) + (1.0 - beta2) * g * g
        p = p - lr * (m1 / bc1) / (np.sqrt(v1 / bc2) + eps)
        out_p.append(p)
        out_m.append(m1)
        out_v.append(v1)
    return out_p, out_m, out_v, norm
