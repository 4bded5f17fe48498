"""The DPO step through the C ABI: the reference model is the streamed frozen
base with the adapters off.  Oracle parity (sequence log-probabilities, loss,
adapter gradients), the fused and the separate reference pass giving the same
bits, streamed against resident, copy accounting and argument checks."""
import numpy as np
import pytest
import torch

from layer_streamed_frozen_amd import binding as B
from layer_streamed_frozen_amd import store as S
from layer_streamed_frozen_amd import synth
from oracle import dpo as D
from tests._util import TOL, report, report_sum
from tests.test_gpu_layer import SMALL, oracle_layer_weights, oracle_shape
from tests.test_gpu_stack import Setup

pytestmark = pytest.mark.gpu

BETA = 0.1


class DpoSetup(Setup):
    def __init__(self, shape, n_layers, vocab, pairs, seq, prefix, prompt_len=None, **kw):
        super().__init__(shape, n_layers, vocab, 2 * pairs, seq, prefix, **kw)
        self.ids_np = synth.preference_pairs(prefix + ".pairs", pairs, seq, vocab,
                                             seq // 2 if prompt_len is None else prompt_len)
        self.ids = torch.from_numpy(self.ids_np).cuda()

    def dpo(self, fused=True, mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS, loss_scale=1.0, beta=BETA):
        self.stack.dpo_step(self.ids, self.emb, self.fnorm, self.head, self.lora.array(), beta=beta, fused=fused,
                            mode=mode, loss_scale=loss_scale)
        torch.cuda.synchronize()

    def snapshot(self):
        return super().snapshot() + (self.stack.seq_logp.clone(),)

    def dpo_oracle(self):
        layers = [oracle_layer_weights(self.wfn(i), self.fmt) for i in range(self.L)]
        loras = [self.lora.numpy(i) for i in range(self.L)]
        return D.dpo_step(self.ids_np, self.emb_np, layers, loras, self.fnorm_np.astype(np.float64),
                          self.head_np.astype(np.float64), oracle_shape(self.shape), beta=BETA)


def same(a, b):
    if not (torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[3], b[3])):
        return False
    for x, y in zip(a[2], b[2]):
        for n in x:
            if not (torch.equal(x[n][0], y[n][0]) and torch.equal(x[n][1], y[n][1])):
                return False
    return True


@pytest.fixture(scope="module")
def pair():
    s = DpoSetup(SMALL, 3, 1024, 2, 96, "dpo")
    # adapters 30x the initial scale, so that policy and reference differ by
    # far more than the bf16 noise of a 95-term log-probability sum
    for i in range(s.L):
        for n in s.lora.targets:
            s.lora.B[i][n].mul_(30.0)
    return s


def test_dpo_matches_oracle(pair):
    pair.dpo()
    ref = pair.dpo_oracle()
    lp = pair.stack.seq_logp.double().cpu().numpy()
    loss = float(pair.stack.loss.item())
    h_gpu = (lp[0, :2] - lp[1, :2]) - (lp[0, 2:] - lp[1, 2:])
    h_ref = (ref["lp_pi"][:2] - ref["lp_ref"][:2]) - (ref["lp_pi"][2:] - ref["lp_ref"][2:])
    print(f"  lp_pi  gpu={lp[0]} oracle={ref['lp_pi']}", flush=True)
    print(f"  lp_ref gpu={lp[1]} oracle={ref['lp_ref']}", flush=True)
    print(f"  h gpu={h_gpu} oracle={h_ref}; loss gpu={loss:.7f} oracle={ref['loss']:.7f}", flush=True)
    # the loss the kernels report is mean softplus(-beta h) of the log-probabilities they report
    assert abs(loss - float(np.mean(np.logaddexp(0.0, -BETA * h_gpu)))) < 1e-5
    # sequence log-probabilities: sums of 95 bf16-activation log-softmax terms
    assert report("lp_pi", lp[0], ref["lp_pi"]) < TOL
    assert report("lp_ref", lp[1], ref["lp_ref"]) < TOL
    # the loss moves by at most beta/2 per unit of h error; h errors of a few
    # tenths (correlated bf16 rounding in policy and reference) stay below 2e-2
    assert abs(loss - ref["loss"]) < BETA / 2 * max(0.2, 2 * float(np.max(np.abs(h_gpu - h_ref)))) + 1e-6
    assert abs(loss - ref["loss"]) < 2e-2
    # the preference margins themselves
    assert float(np.max(np.abs(h_gpu - h_ref))) <= 0.05 * float(np.max(np.abs(h_ref))) + 0.1
    assert report("logits", pair.stack.logits.double().cpu().numpy(), ref["logits"]) < TOL
    for i in range(pair.L):
        g = pair.lora.grads_numpy(i)
        for n in S.PROJ:
            assert report(f"L{i}.dA_{n}", g[n][0], ref["grads"][i][n][0]) < TOL
            assert report(f"L{i}.dB_{n}", g[n][1], ref["grads"][i][n][1]) < TOL


def test_fused_and_separate_reference_pass_bit_equal(pair):
    pair.dpo(fused=True)
    a = pair.snapshot()
    pair.dpo(fused=False)
    assert same(a, pair.snapshot())


def test_dpo_streamed_equals_resident_bitwise(pair):
    pair.dpo(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    a = pair.snapshot()
    pair.dpo(mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    assert same(a, pair.snapshot())
    pair.dpo(fused=False, mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    assert same(a, pair.snapshot())


def test_dpo_forward_only_gives_same_loss(pair):
    pair.dpo()
    a = pair.snapshot()
    pair.dpo(mode=B.MODE_STREAMED | B.MODE_FWD_ONLY)
    assert torch.equal(a[1], pair.stack.loss) and torch.equal(a[3], pair.stack.seq_logp)


def test_zero_adapter_output_gives_ln2_and_equal_logprobs():
    s = DpoSetup(SMALL, 2, 512, 1, 40, "dpo0", targets=("q", "down"))
    for i in range(s.L):
        for n in s.lora.targets:
            s.lora.B[i][n].zero_()
    s.dpo()
    lp = s.stack.seq_logp
    assert torch.equal(lp[0], lp[1])
    assert abs(float(s.stack.loss.item()) - np.log(2.0)) < 1e-6
    # with B = 0 only dB can be non-zero; dA is exactly zero
    for i in range(s.L):
        for n in s.lora.targets:
            assert float(s.lora.dA[i][n].abs().max()) == 0.0
            assert float(s.lora.dB[i][n].abs().max()) > 0.0


def test_dpo_copy_accounting():
    s = DpoSetup(SMALL, 4, 512, 1, 48, "dpocnt")
    L = s.L
    B.stack_reset_stats(s.stack.handle)
    s.dpo(fused=True)
    assert s.stack.stats().copies == 2 * L - 2   # one read per layer per walk, turn reuse as SFT
    B.stack_reset_stats(s.stack.handle)
    s.dpo(fused=True)
    assert s.stack.stats().copies == 2 * L - 4
    a = s.snapshot()
    B.stack_reset_stats(s.stack.handle)
    s.dpo(fused=False)
    assert s.stack.stats().copies == 3 * L - 4   # the separate reference pass reads the stack once more
    assert same(a, s.snapshot())


def test_dpo_bad_arguments():
    s = DpoSetup(SMALL, 2, 256, 1, 16, "dpobad")
    with pytest.raises(B.LsfError) as e:
        s.dpo(beta=0.0)
    assert e.value.status == B.LSF_ERR_INVALID_ARG
    odd = S.Stack(SMALL, s.store, 3, 16, 256)
    ids = torch.zeros((3, 16), dtype=torch.int32, device="cuda")
    with pytest.raises(B.LsfError) as e:
        odd.dpo_step(ids, s.emb, s.fnorm, s.head, s.lora.array())
    assert e.value.status == B.LSF_ERR_SHAPE
    odd.close()


def test_dpo_with_kept_activations_gives_the_same_bits(pair):
    pair.dpo()
    a = pair.snapshot()
    kept = S.Stack(SMALL, pair.store, 4, 96, 1024, keep_activations=True)
    for fused in (True, False):
        kept.dpo_step(pair.ids, pair.emb, pair.fnorm, pair.head, pair.lora.array(), beta=BETA, fused=fused,
                      mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
        torch.cuda.synchronize()
        got = (kept.logits.clone(), kept.loss.clone(),
               [{n: (pair.lora.dA[i][n].clone(), pair.lora.dB[i][n].clone()) for n in pair.lora.targets}
                for i in range(pair.L)], kept.seq_logp.clone())
        assert same(a, got)
    kept.close()


def _oracle_grads_at(s, *dlps):
    """The oracle's policy forward, then one backward per vector of
    per-sequence factors dloss/dl(s) = dlp (the DPO gradient is linear in
    them)."""
    from oracle import model as M
    layers = [oracle_layer_weights(s.wfn(i), s.fmt) for i in range(s.L)]
    loras = [s.lora.numpy(i) for i in range(s.L)]
    oc = oracle_shape(s.shape)
    fn, hd = s.fnorm_np.astype(np.float64), s.head_np.astype(np.float64)
    logits, state = M.stack_forward(s.ids_np, s.emb_np, layers, loras, fn, hd, oc)
    Bsz, T = s.ids_np.shape
    labels, valid = M.shifted_labels(s.ids_np)
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    p[np.arange(p.shape[0]), labels] -= 1.0                  # softmax - onehot
    del e, logits
    out = []
    for dlp in dlps:
        dlogits = -np.repeat(np.asarray(dlp, np.float64), T)[:, None] * p
        dlogits[~valid] = 0.0
        grads, _ = M.stack_backward(dlogits, layers, loras, fn, hd, oc, state)
        out.append(grads)
        del dlogits
    return out[0] if len(out) == 1 else out


def test_dpo_at_8b_shapes_full_vocabulary_matches_oracle():
    # Two Llama-3.1-8B-shaped layers, the 128256-entry vocabulary, 2 pairs of
    # 512 tokens sharing a 256-token prompt (the preference workload):
    # sequence log-probabilities, loss and logits against the oracle's DPO step,
    # so the multi-pass per-sequence sums (511 labelled rows) and the
    # full-vocabulary head are covered.  Adapters at their initial scale: the
    # preference margins h are then of the order of the bf16 noise of 511-term
    # sums (about 0.5 here), and each pair's gradient factor beta sigma(-beta h)
    # / P moves with that noise (a few percent), so the adapter gradients are
    # compared with the oracle's backward at the factors the GPU derived from
    # its own log-probabilities.  The loss is the same function of the
    # log-probabilities: a difference of four sums near -6400 feeds it, so
    # its relative error is about 400 times theirs and is not held to the
    # 2e-2 bound.  Instead each sequence log-probability (a sum of 511
    # same-sign terms) must be within one bf16 unit roundoff (2^-9) of the
    # oracle's relatively, and the loss within what that allows: it is
    # beta-Lipschitz in every margin h, so |dloss| <= beta * mean |dh|.
    s = DpoSetup(S.LLAMA8B, 2, 128256, 2, 512, "dpo8b", random_norms=False)
    s.dpo()
    a = s.snapshot()
    s.dpo(mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    assert same(a, s.snapshot())
    print("  oracle ...", flush=True)
    ref = s.dpo_oracle()
    lp = s.stack.seq_logp.double().cpu().numpy()
    loss = float(s.stack.loss.item())
    h_gpu = (lp[0, :2] - lp[1, :2]) - (lp[0, 2:] - lp[1, 2:])
    h_ref = (ref["lp_pi"][:2] - ref["lp_ref"][:2]) - (ref["lp_pi"][2:] - ref["lp_ref"][2:])
    print(f"  lp_pi  gpu={lp[0]} oracle={ref['lp_pi']}", flush=True)
    print(f"  lp_ref gpu={lp[1]} oracle={ref['lp_ref']}", flush=True)
    print(f"  h gpu={h_gpu} oracle={h_ref}; loss gpu={loss:.7f} oracle={ref['loss']:.7f}", flush=True)
    assert abs(loss - float(np.mean(np.logaddexp(0.0, -BETA * h_gpu)))) < 1e-5
    assert report("lp_pi", lp[0], ref["lp_pi"]) < TOL
    assert report("lp_ref", lp[1], ref["lp_ref"]) < TOL
    for got, want in ((lp[0], ref["lp_pi"]), (lp[1], ref["lp_ref"])):
        assert np.max(np.abs(got - want) / np.abs(want)) < 2.0 ** -9
    assert abs(loss - ref["loss"]) <= BETA * float(np.mean(np.abs(h_gpu - h_ref))) + 1e-5
    assert report("logits", s.stack.logits.double().cpu().numpy(), ref["logits"]) < TOL
    _, dlp_gpu = D.dpo_loss(lp[0], lp[1], BETA)
    _, dlp_ref = D.dpo_loss(ref["lp_pi"], ref["lp_ref"], BETA)
    print(f"  per-sequence factors gpu={dlp_gpu} oracle={dlp_ref}", flush=True)
    # The gradient is the chosen sequences' part plus the rejected ones', of
    # opposite sign over a shared prompt; the oracle also gives the chosen
    # part alone, and each part held to TOL bounds the error of the sum.
    chosen = np.array([1.0, 1.0, 0.0, 0.0]) * dlp_gpu
    grads, grads_c = _oracle_grads_at(s, dlp_gpu, chosen)
    for i in range(s.L):
        g = s.lora.grads_numpy(i)
        for n in S.PROJ:
            for k, nm in ((0, "dA"), (1, "dB")):
                assert report_sum(f"L{i}.{nm}_{n}", g[n][k], grads[i][n][k], grads_c[i][n][k]) < TOL
    # for the record: the same gradients against the oracle's own factors
    for n in ("q", "down"):
        print(f"  (at the oracle's factors) L1.dA_{n} rel_fro="
              f"{np.linalg.norm(s.lora.grads_numpy(1)[n][0] - ref['grads'][1][n][0]) / np.linalg.norm(ref['grads'][1][n][0]):.3e}",
              flush=True)
    s.stack.close()
