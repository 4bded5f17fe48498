"""The streamed stack step through the C ABI: oracle parity, the pages'
bit-equality of streamed and resident runs, copy accounting, accumulation,
forward-only mode and the pinned / pageable host-store rules."""
import numpy as np
import pytest
import torch

from layer_streamed_frozen_amd import binding as B
from layer_streamed_frozen_amd import store as S
from layer_streamed_frozen_amd import synth
from oracle import model as M
from oracle import nf4 as onf4
from tests._util import TOL, bf16_tensor_to_np, report
from tests.test_gpu_layer import LARGE, SMALL, bf16_weights, oracle_layer_weights, oracle_shape

pytestmark = pytest.mark.gpu


def bf16_param(name, shape, std):
    vals, bits = synth.bf16_exact(synth.normal(name, shape, std))
    return vals, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


class Setup:
    def __init__(self, shape, n_layers, vocab, batch, seq, prefix, resident=True, targets=S.PROJ, flags=0,
                 pinned=True, random_norms=True, fmt=B.FMT_NF4):
        print(f"[stack] {prefix} L={n_layers} V={vocab} B={batch} S={seq}", flush=True)
        self.shape, self.L, self.V, self.batch, self.seq = shape, n_layers, vocab, batch, seq
        self.prefix = prefix

        def wfn(i):
            W = S.layer_weights_fp32(f"{prefix}.layer{i}", shape)
            if random_norms:
                W.update(S.random_norms(f"{prefix}.layer{i}", shape))
            return bf16_weights(W) if fmt == B.FMT_BF16 else W

        self.wfn = wfn
        self.fmt = fmt
        self.store = S.Store(shape, n_layers, fmt=fmt, resident=resident, weights_fn=wfn, pinned=pinned)
        self.lora = S.LoraSet(shape, n_layers, targets=targets, prefix=prefix + ".lora")
        H = shape.hidden
        self.emb_np, self.emb = bf16_param(prefix + ".embed", (vocab, H), 1.0)
        self.head_np, self.head = bf16_param(prefix + ".head", (vocab, H), 0.02)
        fn = np.full(H, 0x3F80, np.uint16)
        self.fnorm_np = onf4.bf16_to_f32(fn)
        self.fnorm = torch.from_numpy(fn.view(np.int16)).view(torch.bfloat16).cuda()
        self.ids_np = synth.token_ids(prefix + ".ids", (batch, seq), vocab)
        self.ids = torch.from_numpy(self.ids_np).cuda()
        self.stack = S.Stack(shape, self.store, batch, seq, vocab, flags=flags)

    def step(self, mode=B.MODE_STREAMED, loss_scale=1.0, enabled=True, ids=None):
        arr = self.lora.array(enabled=enabled)
        self.stack.step(self.ids if ids is None else ids, self.emb, self.fnorm, self.head, arr, mode=mode,
                        loss_scale=loss_scale)
        torch.cuda.synchronize()

    def snapshot(self):
        g = [{n: (self.lora.dA[i][n].clone(), self.lora.dB[i][n].clone()) for n in self.lora.targets}
             for i in range(self.L)]
        return self.stack.logits.clone(), self.stack.loss.clone(), g

    def oracle(self, loss_scale=1.0, ids=None):
        layers = [oracle_layer_weights(self.wfn(i), self.fmt) for i in range(self.L)]
        loras = [self.lora.numpy(i) for i in range(self.L)]
        return M.stack_step(self.ids_np if ids is None else ids, self.emb_np, layers, loras,
                            self.fnorm_np.astype(np.float64), self.head_np.astype(np.float64),
                            oracle_shape(self.shape), loss_scale=loss_scale)


def same(a, b):
    la, sa, ga = a
    lb, sb, gb = b
    if not (torch.equal(la, lb) and torch.equal(sa, sb)):
        return False
    for x, y in zip(ga, gb):
        for n in x:
            if not (torch.equal(x[n][0], y[n][0]) and torch.equal(x[n][1], y[n][1])):
                return False
    return True


@pytest.fixture(scope="module")
def small():
    return Setup(SMALL, 3, 1024, 2, 100, "ss")


def test_small_stack_matches_oracle(small):
    small.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    ref = small.oracle()
    loss = float(small.stack.loss.item())
    print(f"  loss gpu={loss:.6f} oracle={ref['loss']:.6f}", flush=True)
    assert abs(loss - ref["loss"]) / abs(ref["loss"]) < TOL
    assert report("logits", small.stack.logits.double().cpu().numpy(), ref["logits"]) < TOL
    for i in range(small.L):
        g = small.lora.grads_numpy(i)
        for n in S.PROJ:
            assert report(f"L{i}.dA_{n}", g[n][0], ref["grads"][i][n][0]) < TOL
            assert report(f"L{i}.dB_{n}", g[n][1], ref["grads"][i][n][1]) < TOL


def test_streamed_equals_resident_bitwise(small):
    small.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    a = small.snapshot()
    small.step(mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    b = small.snapshot()
    print(f"  max|logit diff| = {float((a[0] - b[0]).abs().max()):.1f}", flush=True)
    assert same(a, b)


def test_forward_and_backward_bit_equal_separately(small):
    # forward claim: logits and loss of a forward-only step
    small.step(mode=B.MODE_STREAMED | B.MODE_FWD_ONLY)
    fa = (small.stack.logits.clone(), small.stack.loss.clone())
    small.step(mode=B.MODE_RESIDENT | B.MODE_FWD_ONLY)
    assert torch.equal(fa[0], small.stack.logits) and torch.equal(fa[1], small.stack.loss)
    # backward claim: the gradients
    small.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    a = small.snapshot()
    small.step(mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    assert same(a, small.snapshot())


def test_run_to_run_determinism(small):
    small.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    a = small.snapshot()
    small.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    assert same(a, small.snapshot())


def test_copy_accounting():
    s = Setup(SMALL, 4, 512, 1, 48, "cnt")
    L = s.L
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    st = s.stack.stats()
    assert st.steps == 1
    assert st.copies == 2 * L - 2                # the two layers resident at the turn are reused
    assert st.bytes == st.copies * s.store.blob_bytes()
    a = s.snapshot()
    B.stack_reset_stats(s.stack.handle)
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    assert s.stack.stats().copies == 2 * L - 4   # layers 0 and 1 are still resident from the last step
    assert same(a, s.snapshot())
    B.stack_reset_stats(s.stack.handle)
    s.step(mode=B.MODE_STREAMED | B.MODE_FWD_ONLY)
    assert s.stack.stats().copies == L - 2
    B.stack_reset_stats(s.stack.handle)
    s.step(mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    assert s.stack.stats().copies == 0
    assert same(a, s.snapshot())
    # after a forward-only step the buffers hold layers L-2 and L-1: layer 0 must be copied again
    B.stack_reset_stats(s.stack.handle)
    s.step(mode=B.MODE_STREAMED | B.MODE_FWD_ONLY)
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    assert same(a, s.snapshot())


def test_no_turn_reuse_and_timing_give_same_bits():
    s = Setup(SMALL, 3, 1024, 1, 64, "nt", flags=B.STACK_NO_TURN_REUSE | B.STACK_TIMING)
    B.stack_reset_stats(s.stack.handle)
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    st = s.stack.stats()
    assert st.copies == 2 * s.L
    assert st.copy_ms > 0.0
    assert st.kernel_launches[B.KERNELS.index("gate_up_fwd")] == 2 * s.L  # forward + recompute
    assert st.kernel_launches[B.KERNELS.index("down_bwd")] == s.L
    a = s.snapshot()
    s.step(mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    assert same(a, s.snapshot())


@pytest.mark.parametrize("flags", [0, B.STACK_ONE_COPY_STREAM, B.STACK_TIMING, B.STACK_ONE_COPY_STREAM | B.STACK_TIMING])
def test_one_and_two_copy_streams_give_same_bits(flags):
    # Each layer copy as two halves on two copy streams (the default) or as one
    # transfer: the same bytes in the buffers, so the streamed step equals the
    # resident one bit for bit either way, over two steps (turn and step
    # boundary reuse included); with timing, every copy is counted once.
    s = Setup(SMALL, 3, 1024, 1, 64, "cs", flags=flags)
    B.stack_reset_stats(s.stack.handle)
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    st = s.stack.stats()
    assert st.copies == (2 * s.L - 2) + (2 * s.L - 4)
    if flags & B.STACK_TIMING:
        assert st.copy_ms > 0.0
    a = s.snapshot()
    s.step(mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    assert same(a, s.snapshot())


def test_gradient_accumulation_matches_oracle():
    s = Setup(SMALL, 2, 512, 1, 80, "acc", random_norms=False)
    ids2 = synth.token_ids("acc.ids2", (1, 80), 512)
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS, loss_scale=0.5)
    s.step(mode=B.MODE_STREAMED, loss_scale=0.5, ids=torch.from_numpy(ids2).cuda())
    r1 = s.oracle(loss_scale=0.5)
    r2 = s.oracle(loss_scale=0.5, ids=ids2)
    for i in range(s.L):
        g = s.lora.grads_numpy(i)
        for n in ("q", "o", "down"):
            assert report(f"L{i}.dA_{n}", g[n][0], r1["grads"][i][n][0] + r2["grads"][i][n][0]) < TOL
            assert report(f"L{i}.dB_{n}", g[n][1], r1["grads"][i][n][1] + r2["grads"][i][n][1]) < TOL


def test_accumulated_walk_equals_sequential_micro_batches():
    # Three micro-batches: one stream_stack_accum_step (each layer copied once
    # per direction for all three) against three stream_stack_step calls.
    n = 3
    s = Setup(SMALL, 4, 512, 2, 64, "accw")
    ids = [torch.from_numpy(synth.token_ids(f"accw.ids{m}", (2, 64), 512)).cuda() for m in range(n)]
    arr = s.lora.array()
    for m in range(n):
        mode = B.MODE_STREAMED | (B.MODE_ZERO_GRADS if m == 0 else 0)
        s.stack.step(ids[m], s.emb, s.fnorm, s.head, arr, mode=mode, loss_scale=1.0 / n)
    torch.cuda.synchronize()
    ref = s.snapshot()
    ref_ckpt = s.stack.ckpt.clone()

    def run(mode, keep=False):
        acc = S.Stack(SMALL, s.store, 2, 64, 512, n_micro=n, keep_activations=keep)
        B.stack_reset_stats(acc.handle)
        acc.accum_step(ids, s.emb, s.fnorm, s.head, arr, mode=mode)
        torch.cuda.synchronize()
        g = [{k: (s.lora.dA[i][k].clone(), s.lora.dB[i][k].clone()) for k in s.lora.targets} for i in range(s.L)]
        out = (acc.logits.clone(), acc.loss.clone(), g)
        st = acc.stats()
        ck = acc.ckpts[n - 1].clone()
        acc.close()
        return out, st, ck

    got, st, ck = run(B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    assert st.steps == n
    assert st.copies == 2 * s.L - 2       # once per direction, not once per micro-batch
    assert same(ref, got)                 # last micro-batch's logits and loss, every gradient
    assert torch.equal(ck, ref_ckpt)
    got_r, st_r, _ = run(B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    assert st_r.copies == 0 and same(ref, got_r)
    got_k, _, _ = run(B.MODE_STREAMED | B.MODE_ZERO_GRADS, keep=True)
    assert same(ref, got_k)


def test_accumulated_walk_argument_errors():
    s = Setup(SMALL, 2, 256, 1, 32, "accx")
    arr = s.lora.array()
    with pytest.raises(B.LsfError) as e:
        B.stream_stack_accum_step(s.stack.handle, [])
    assert e.value.status == B.LSF_ERR_INVALID_ARG
    # a workspace sized for one micro-batch is too small for two
    io = s.stack._io(s.ids, s.emb, s.fnorm, s.head, arr, B.MODE_STREAMED, 0.5)
    with pytest.raises(B.LsfError) as e:
        B.stream_stack_accum_step(s.stack.handle, [io, io])
    assert e.value.status == B.LSF_ERR_WORKSPACE
    assert B.stack_accum_workspace_bytes(s.stack.cfg, 256, 2, 2) > B.stack_workspace_bytes(s.stack.cfg, 256, 2)
    assert B.stack_accum_workspace_bytes(s.stack.cfg, 256, 2, 1) == B.stack_workspace_bytes(s.stack.cfg, 256, 2)
    assert B.stack_accum_workspace_bytes(s.stack.cfg, 256, 2, 0) == 0


def test_adapters_disabled_changes_only_through_lora():
    s = Setup(SMALL, 2, 512, 1, 48, "dis", targets=("q", "v"))
    s.step(mode=B.MODE_STREAMED | B.MODE_FWD_ONLY, enabled=False)
    layers = [oracle_layer_weights(s.wfn(i)) for i in range(s.L)]
    logits, _ = M.stack_forward(s.ids_np, s.emb_np, layers, [None] * s.L,
                                s.fnorm_np.astype(np.float64), s.head_np.astype(np.float64), oracle_shape(s.shape))
    assert report("logits", s.stack.logits.double().cpu().numpy(), logits) < TOL


def test_pageable_store_rules():
    st = S.Store(SMALL, 2, resident=False, pinned=False, prefix="pg")
    with pytest.raises(B.LsfError) as e:
        S.Stack(SMALL, st, 1, 32, 256)
    assert e.value.status == B.LSF_ERR_NOT_PINNED
    # accepted with the explicit flag (the slow fallback); results unchanged
    pinned = S.Store(SMALL, 2, resident=False, pinned=True, prefix="pg")
    lora = S.LoraSet(SMALL, 2, prefix="pg.lora")
    emb = bf16_param("pg.embed", (256, SMALL.hidden), 1.0)[1]
    head = bf16_param("pg.head", (256, SMALL.hidden), 0.02)[1]
    fn = torch.ones(SMALL.hidden, dtype=torch.bfloat16, device="cuda")
    ids = torch.from_numpy(synth.token_ids("pg.ids", (1, 32), 256)).cuda()
    outs = []
    for store, flags in ((st, B.STACK_ALLOW_PAGEABLE), (pinned, 0)):
        sk = S.Stack(SMALL, store, 1, 32, 256, flags=flags)
        sk.step(ids, emb, fn, head, lora.array(), mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
        torch.cuda.synchronize()
        outs.append((sk.logits.clone(), lora.dA[1]["q"].clone()))
        sk.close()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_bad_arguments_are_rejected():
    cfg = SMALL.cfg(1, 16)
    d = B.StackDesc()
    d.n_layers = 0
    with pytest.raises(B.LsfError) as e:
        B.stack_create(cfg, d)
    assert e.value.status == B.LSF_ERR_INVALID_ARG


def test_full_8b_shapes_two_layers_match_oracle():
    # Llama-3.1-8B-shaped layers and the full 128256-entry vocabulary, seq 512
    s = Setup(S.LLAMA8B, 2, 128256, 1, 512, "s8b2", random_norms=False)
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    a = s.snapshot()
    s.step(mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    assert same(a, s.snapshot())
    ref = s.oracle()
    loss = float(s.stack.loss.item())
    print(f"  loss gpu={loss:.6f} oracle={ref['loss']:.6f}", flush=True)
    assert abs(loss - ref["loss"]) / abs(ref["loss"]) < TOL
    assert report("logits", s.stack.logits.double().cpu().numpy(), ref["logits"]) < TOL
    for i in range(s.L):
        g = s.lora.grads_numpy(i)
        for n in S.PROJ:
            assert report(f"L{i}.dA_{n}", g[n][0], ref["grads"][i][n][0]) < TOL
            assert report(f"L{i}.dB_{n}", g[n][1], ref["grads"][i][n][1]) < TOL


def test_full_8b_shapes_batch4_two_layers_match_oracle():
    # The batch-4 micro-batch of the accumulation workload (4 x 512 tokens) on
    # two 8B-shaped layers with the full vocabulary: the head at 2048 x 128256,
    # the loss, logits and every adapter gradient against the oracle.
    s = Setup(S.LLAMA8B, 2, 128256, 4, 512, "s8b4", random_norms=False)
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS, loss_scale=0.25)
    print("  oracle ...", flush=True)
    ref = s.oracle(loss_scale=0.25)
    loss = float(s.stack.loss.item())
    print(f"  loss gpu={loss:.6f} oracle={ref['loss']:.6f}", flush=True)
    assert abs(loss - ref["loss"]) / abs(ref["loss"]) < TOL
    assert report("logits", s.stack.logits.double().cpu().numpy(), ref["logits"]) < TOL
    for i in range(s.L):
        g = s.lora.grads_numpy(i)
        for n in S.PROJ:
            assert report(f"L{i}.dA_{n}", g[n][0], ref["grads"][i][n][0]) < TOL
            assert report(f"L{i}.dB_{n}", g[n][1], ref["grads"][i][n][1]) < TOL
    s.stack.close()


def test_layers_above_165_mib_stream_bit_equal():
    # two 274 MB layers (hidden 5120, intermediate 27648): every copy moves more
    # than 165 MiB, and the streamed step must give the resident step's bits,
    # forward and backward
    s = Setup(LARGE, 2, 1024, 1, 512, "s14b", resident=True, random_norms=False)
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    a = s.snapshot()
    st = s.stack.stats()
    assert st.copies == 2 and st.bytes == 2 * s.store.blob_bytes() and s.store.blob_bytes() > 165 * 2**20
    s.step(mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    assert same(a, s.snapshot())
    assert all(torch.isfinite(a[2][i][n][k]).all() for i in range(2) for n in S.PROJ for k in range(2))
    s.stack.close()


def test_out_of_range_ids_set_the_status_word():
    s = Setup(SMALL, 2, 512, 2, 40, "badid")
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    assert s.stack.ids_were_valid()
    good_logits = s.stack.logits.clone()
    for bad in (512, -1, 1 << 30):
        ids = s.ids.clone()
        ids[1, 7] = bad
        s.stack.clear_id_status()
        s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS, ids=ids)
        assert not s.stack.ids_were_valid(), bad
        # the bad position embeds as zeros; the rows of the other sequence are untouched
        assert torch.count_nonzero(s.stack.ckpt[0, 40 + 7]) == 0
        assert torch.equal(s.stack.logits[:40], good_logits[:40])
        assert torch.isfinite(s.stack.loss).all()
    s.stack.clear_id_status()
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    assert s.stack.ids_were_valid() and torch.equal(s.stack.logits, good_logits)


@pytest.mark.parametrize("fmt", [B.FMT_NF4_DQ, B.FMT_BF16])
def test_other_base_formats_stream_bit_equal_and_match_oracle(fmt):
    s = Setup(SMALL, 3, 512, 1, 72, f"fmt{fmt}", fmt=fmt)
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    a = s.snapshot()
    s.step(mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    assert same(a, s.snapshot())
    ref = s.oracle()
    assert abs(float(s.stack.loss.item()) - ref["loss"]) / abs(ref["loss"]) < TOL
    assert report("logits", s.stack.logits.double().cpu().numpy(), ref["logits"]) < TOL
    for i in range(s.L):
        g = s.lora.grads_numpy(i)
        for n in ("q", "o", "gate", "down"):
            assert report(f"L{i}.dA_{n}", g[n][0], ref["grads"][i][n][0]) < TOL
            assert report(f"L{i}.dB_{n}", g[n][1], ref["grads"][i][n][1]) < TOL


def test_single_kernel_class_timing_and_unknown_flags():
    k = B.KERNELS.index("gate_up_fwd")
    s = Setup(SMALL, 2, 512, 1, 48, "tk", flags=B.STACK_TIME_KERNEL(k))
    B.stack_reset_stats(s.stack.handle)
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    st = s.stack.stats()
    assert st.kernel_launches[k] == 2 * s.L      # forward + recompute
    assert all(st.kernel_launches[i] == 0 for i in range(len(B.KERNELS)) if i != k)
    assert st.copy_ms == 0.0 and st.wait_ms == 0.0
    with pytest.raises(B.LsfError) as e:
        S.Stack(SMALL, s.store, 1, 48, 512, flags=1 << 30)
    assert e.value.status == B.LSF_ERR_INVALID_ARG


def test_kept_activations_give_the_same_bits():
    s = Setup(SMALL, 3, 512, 2, 64, "keep")
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    a = s.snapshot()
    kept = S.Stack(SMALL, s.store, 2, 64, 512, keep_activations=True)
    for mode in (B.MODE_STREAMED, B.MODE_RESIDENT):
        kept.step(s.ids, s.emb, s.fnorm, s.head, s.lora.array(), mode=mode | B.MODE_ZERO_GRADS)
        torch.cuda.synchronize()
        got = (kept.logits.clone(), kept.loss.clone(),
               [{n: (s.lora.dA[i][n].clone(), s.lora.dB[i][n].clone()) for n in s.lora.targets}
                for i in range(s.L)])
        assert same(a, got)
    # the layers are still read twice per micro-batch
    B.stack_reset_stats(kept.handle)
    kept.step(s.ids, s.emb, s.fnorm, s.head, s.lora.array(), mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    torch.cuda.synchronize()
    assert kept.stats().copies == 2 * s.L - 4
    # an arena that is too small is refused before anything runs
    io = kept._io(s.ids, s.emb, s.fnorm, s.head, s.lora.array(), B.MODE_STREAMED, 1.0)
    io.act_bytes = kept.act.numel() - 256
    with pytest.raises(B.LsfError) as e:
        B.stream_stack_step(kept.handle, io)
    assert e.value.status == B.LSF_ERR_WORKSPACE
    kept.close()


def test_bench_configuration_32_layers_full_vocabulary():
    # The configuration bench.py times: 32 Llama-3.1-8B-shaped layers (the same
    # seeded weights), vocabulary 128256, one sequence of 512 tokens.  At this
    # size the oracle checks the first layer's output (from the embedding and
    # layer 0's weights alone); the whole step is checked by the bit-equality of
    # the streamed and the resident runs and by the copy count.
    shape = S.LLAMA8B
    L, V, seq = 32, 128256, 512
    print(f"[stack] bench configuration L={L} V={V} seq={seq}", flush=True)
    store = S.Store(shape, L, resident=True, pinned=True, weights_fn=lambda i: S.layer_weights_fp32(f"layer{i}", shape))
    lora = S.LoraSet(shape, L)
    H = shape.hidden
    emb_np, emb = bf16_param("embed", (V, H), 1.0)
    head_np, head = bf16_param("lm_head", (V, H), 0.02)
    fnorm = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    ids_np = synth.token_ids("ids0", (1, seq), V)
    ids = torch.from_numpy(ids_np).cuda()
    stack = S.Stack(shape, store, 1, seq, V)
    arr = lora.array()

    def run(mode):
        stack.step(ids, emb, fnorm, head, arr, mode=mode | B.MODE_ZERO_GRADS)
        torch.cuda.synchronize()
        return (stack.logits.clone(), stack.loss.clone(),
                [{n: (lora.dA[i][n].clone(), lora.dB[i][n].clone()) for n in lora.targets} for i in range(L)])

    n0 = B.gemm_wide_launch_count()
    a = run(B.MODE_STREAMED)
    # gate|up forward and recompute, the down forward (split-K), and the
    # gate|up and down input gradients of every layer on the ping-pong kernels
    assert B.gemm_wide_launch_count() - n0 == 5 * L
    layer1 = stack.ckpt[1].clone()
    B.stack_reset_stats(stack.handle)
    a2 = run(B.MODE_STREAMED)
    assert stack.stats().copies == 2 * L - 4
    assert same(a, a2)
    assert same(a, run(B.MODE_RESIDENT))
    loss = float(a[1].item())
    print(f"  loss {loss:.4f} (ln V = {np.log(V):.4f})", flush=True)
    assert np.isfinite(loss) and abs(loss - np.log(V)) < 1.0
    # layer 0 against the oracle, from the ids and the embedding
    x = emb_np.astype(np.float64)[ids_np]
    W0 = oracle_layer_weights(S.layer_weights_fp32("layer0", shape))
    y, _ = M.layer_fwd(x, W0, lora.numpy(0), oracle_shape(shape))
    assert report("layer0.y", bf16_tensor_to_np(layer1).reshape(1, seq, H), y) < TOL
    stack.close()


def test_accumulated_walk_at_8b_shapes_batch4():
    # The stack4 bench configuration on four 8B-shaped layers: four micro-batches
    # of 4 x 512 tokens, vocabulary 128256.  One accumulated walk gives the bits
    # of four sequential micro-batch steps (every gradient, the last logits and
    # loss) with 2L - 2 copies; micro-batch by micro-batch takes 2L - 2 for the
    # first and 2L - 4 for each further one (layers 0 and 1 stay resident).
    shape = S.LLAMA8B
    L, V, batch, seq, n = 4, 128256, 4, 512, 4
    print(f"[stack] accumulated walk L={L} V={V} {n} x {batch} x {seq}", flush=True)
    store = S.Store(shape, L, resident=False, pinned=True,
                    weights_fn=lambda i: S.layer_weights_fp32(f"acc8b.layer{i}", shape))
    lora = S.LoraSet(shape, L, prefix="acc8b.lora")
    H = shape.hidden
    _, emb = bf16_param("acc8b.embed", (V, H), 1.0)
    _, head = bf16_param("acc8b.head", (V, H), 0.02)
    fnorm = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    ids = [torch.from_numpy(synth.token_ids(f"acc8b.ids{m}", (batch, seq), V)).cuda() for m in range(n)]
    arr = lora.array()

    def grads():
        return [{k: (lora.dA[i][k].clone(), lora.dB[i][k].clone()) for k in lora.targets} for i in range(L)]

    seq_stack = S.Stack(shape, store, batch, seq, V)
    B.stack_reset_stats(seq_stack.handle)
    for m in range(n):
        mode = B.MODE_STREAMED | (B.MODE_ZERO_GRADS if m == 0 else 0)
        seq_stack.step(ids[m], emb, fnorm, head, arr, mode=mode, loss_scale=1.0 / n)
    torch.cuda.synchronize()
    copies_seq = seq_stack.stats().copies
    ref = (seq_stack.logits.clone(), seq_stack.loss.clone(), grads())
    seq_stack.close()
    del seq_stack
    torch.cuda.empty_cache()

    acc = S.Stack(shape, store, batch, seq, V, n_micro=n)
    B.stack_reset_stats(acc.handle)
    acc.accum_step(ids, emb, fnorm, head, arr, mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    torch.cuda.synchronize()
    st = acc.stats()
    got = (acc.logits.clone(), acc.loss.clone(), grads())
    acc.close()
    print(f"  copies: {copies_seq} micro-batch by micro-batch, {st.copies} in one walk", flush=True)
    assert st.copies == 2 * L - 2
    assert copies_seq == (2 * L - 2) + (n - 1) * (2 * L - 4)
    assert same(ref, got)
    assert all(torch.isfinite(ref[2][i][k][0]).all() for i in range(L) for k in lora.targets)
