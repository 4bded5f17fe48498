"""Oracle: DPO step whose reference model is the frozen base with the
adapters switched off.

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

Source: the project README ("feinterview.poetries.top/.../makazhanalpamys-soup",
the paragraph on preference losses with layer streaming) and the blog
("agentlenshq.com/...", section on DPO support): the DPO reference model is the
same streamed base with its adapter disabled, so no second copy of the weights
is needed.  The pages give no formula; the plain DPO definition is used:

  l(s)  = sum over positions t < T-1 of log softmax(z_t)[ids[t+1]]   (per sequence)
  h_p   = (l_pi(c_p) - l_ref(c_p)) - (l_pi(r_p) - l_ref(r_p))        (per pair p)
  loss  = mean_p  -log sigmoid(beta h_p) = mean_p softplus(-beta h_p),  beta = 0.1

The batch holds the P chosen sequences first, then the P rejected ones.  Only
the policy (adapters on) receives gradients:
  dloss/dl_pi(c_p) = -beta sigmoid(-beta h_p) / P,  dloss/dl_pi(r_p) = -dloss/dl_pi(c_p)
  dloss/dz_t       = dloss/dl(s) (onehot(ids[t+1]) - softmax(z_t))  for labelled t.

Parity: pinned (torch log_softmax for the log-probs, loss = ln 2 when policy
and reference coincide, antisymmetry under swapping chosen and rejected,
fp64 finite differences on a tiny stack).
"""
import numpy as np

from . import model as M


def sequence_logprobs(logits, ids):
    """Sum of next-token log-probabilities per sequence.  logits [B*T, V]."""
    Bsz, T = ids.shape
    labels, valid = M.shifted_labels(ids)
    z = logits
    m = z.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    lp = z[np.arange(z.shape[0]), labels] - lse
    lp[~valid] = 0.0
    return lp.reshape(Bsz, T).sum(axis=1)


def dpo_loss(lp_pi, lp_ref, beta):
    """Returns (loss, dloss/dl_pi per sequence)."""
    P = lp_pi.shape[0] // 2
    h = (lp_pi[:P] - lp_ref[:P]) - (lp_pi[P:] - lp_ref[P:])
    x = -beta * h
    loss = float(np.mean(np.logaddexp(0.0, x)))          # softplus(-beta h)
    sig_neg = 1.0 / (1.0 + np.exp(beta * h))             # sigmoid(-beta h)
    d = np.empty_like(lp_pi)
    d[:P] = -beta * sig_neg / P
    d[P:] = beta * sig_neg / P
    return loss, d


def dpo_step(ids, emb, layers, loras, final_norm, head, cfg, beta=0.1, dtype=np.float64,
             round_boundaries=True):
    """Reference forward (adapters off), policy forward, DPO loss, policy
    backward.  Returns dict(loss, lp_pi, lp_ref, dlogits, grads)."""
    L = len(loras)
    ref_logits, _ = M.stack_forward(ids, emb, layers, [None] * L, final_norm, head, cfg, dtype,
                                    round_boundaries, keep_caches=False)
    logits, state = M.stack_forward(ids, emb, layers, loras, final_norm, head, cfg, dtype, round_boundaries)
    lp_ref = sequence_logprobs(ref_logits, ids)
    lp_pi = sequence_logprobs(logits, ids)
    loss, dlp = dpo_loss(lp_pi, lp_ref, beta)
    Bsz, T = ids.shape
    labels, valid = M.shifted_labels(ids)
    z = logits
    e = np.exp(z - z.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    onehot = np.zeros_like(p)
    onehot[np.arange(z.shape[0]), labels] = 1.0
    coef = np.repeat(dlp, T)[:, None]                    # dloss/dl of the row's sequence
    dlogits = coef * (onehot - p)
    dlogits[~valid] = 0.0
    grads, _ = M.stack_backward(dlogits, layers, loras, final_norm, head, cfg, state, dtype)
    return dict(loss=loss, lp_pi=lp_pi, lp_ref=lp_ref, dlogits=dlogits, grads=grads, logits=logits)
