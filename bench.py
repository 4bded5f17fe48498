"""Throughput of the streamed NF4 + LoRA training step on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload stack1|stack4|dpo|dpo-unfused]
                    [--format nf4|nf4dq|bf16] [--optimizer adamw|adamw8] [--lora-targets all|qv]
                    [--accum-order layer|micro] [--keep-activations] [--no-cpu-baseline]

Workload (default "stack1"): 32 Llama-3.1-8B-shaped decoder layers (hidden
4096, intermediate 14336, 32 query / 8 kv heads of 128, RoPE theta 500000),
frozen base NF4-quantised (64-element blocks, fp32 absmax) in page-locked host
memory, streamed through two device buffers; LoRA rank 16 (alpha 16) on q, k,
v, o, gate, up, down; resident untied bf16 embedding and lm_head over a
128256-token vocabulary; one sequence of 512 random token ids per step;
cross-entropy loss; forward, head, recomputing backward (all LoRA gradients)
and one AdamW update of every adapter per step.  "stack4" is 4 sequences of 512 per micro-batch and 4 micro-batches
(gradient accumulation) per step, by default in one walk over the stack per direction
(each layer copied once for all four micro-batches; ``--accum-order micro`` streams
the stack once per micro-batch instead; both give the same bits).  "dpo" is the preference-loss step: 2
chosen/rejected pairs of 512 tokens (4 sequences, pair p sharing a 256-token
prompt), DPO with beta 0.1, the reference log-probabilities from the same
streamed base with the adapters off, computed in the policy's layer visit
("dpo-unfused": in a separate pass over the stack).  Inputs and weights are
seeded synthetic data.

Prints one JSON line.  ``value`` is tokens per second over the timed steps,
with every input already resident (the frozen store in pinned host memory is
the method's input; its per-step host-to-device traffic is part of the step).
The timed steps carry HIP events around the gate|up forward GEMM only (the
``roofline`` kernel); a diagnostic pass of a few more steps afterwards times
every kernel class and every copy (``kernels``, ``layer_gemms`` and the
copy-engine figures in ``h2d``), since events on every kernel and copy slow
the step by a few percent.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "train tokens/sec (fwd+bwd) streamed 8B-shape NF4+LoRA, seq 512; H2D GB/s"
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBPS = 8000.0
PCIE5_X16_GBPS = 63.0            # theoretical per direction after 128b/130b encoding

# HBM bytes per launch of the gate|up forward GEMM from two rocprofv3 --pmc passes
# (profiles/pmc_traffic_layer8b_seq512.md): FETCH_SIZE 50048.08 KiB scaled by 1.99975
# (the calibration kernel's ratio) + WRITE_SIZE 28692.45 KiB scaled by 1.0.  Valid only
# for the sources of that kernel they were taken on (hash below); otherwise null.
GATE_UP_TRAFFIC_BYTES = (50048.08 * 1.99975 + 28692.45 * 1.0) * 1024
GATE_UP_TRAFFIC_SRC = "9a733b284c9f0cb1"
# Algorithmic bytes of one such launch: NF4 codes 58.72 MB + absmax 7.34 MB + x 4.19 MB +
# LoRA (U, B) 1.9 MB read; a 14.7 MB (forward) or a, g, u 44.0 MB (recompute) written.
GATE_UP_ALGO_BYTES = (58.72 + 7.34 + 4.19 + 1.9 + (14.68 + 44.04) / 2) * 1e6


def gemm_src_hash():
    import hashlib
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "layer_streamed_frozen_amd", "csrc")
    h = hashlib.sha256()
    for f in ("gemm_wide.hip", "common.h", "weight_decode.h"):
        with open(os.path.join(here, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", choices=["stack1", "stack4", "dpo", "dpo-unfused"], default="stack1")
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--format", choices=["nf4", "nf4dq", "bf16"], default="nf4",
                   help="frozen-base storage: NF4 with fp32 absmax, NF4 with 8-bit double-quantised absmax, "
                        "or unquantised bf16")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-timing", action="store_true", help="skip the per-kernel event probes")
    p.add_argument("--timing", choices=["dominant", "all"], default="dominant",
                   help="events in the timed steps: around the gate|up forward GEMM only, or around every "
                        "kernel class and copy")
    p.add_argument("--optimizer", choices=["adamw", "adamw8"], default="adamw",
                   help="adamw8: AdamW with 8-bit block-wise moment states (the pages' paged_adamw_8bit)")
    p.add_argument("--lora-targets", choices=["all", "qv"], default="all",
                   help="qv: adapters on q and v only (the pages' published configuration)")
    p.add_argument("--keep-activations", action="store_true",
                   help="keep every layer's forward intermediates in HBM and skip the recompute in the backward "
                        "walk (each layer is still read twice)")
    p.add_argument("--accum-order", choices=["layer", "micro"], default="layer",
                   help="gradient accumulation: every layer serves all micro-batches in one walk (layer) or "
                        "the stack is walked once per micro-batch (micro)")
    p.add_argument("--diag-steps", type=int, default=5,
                   help="steps of the diagnostic pass that times every kernel class and copy (0: none)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemm_flops(T, shape):
    H, I = shape.hidden, shape.intermediate
    q, kv = shape.n_heads * shape.head_dim, shape.n_kv_heads * shape.head_dim
    n = {"qkv": (q + 2 * kv) * H, "o": H * q, "gate_up": 2 * I * H, "down": H * I}
    return {k: 2.0 * T * v for k, v in n.items()}


def measure_link_peak(torch, nbytes=1 << 30, reps=5):
    """Best pinned host -> device copy rate (GB/s) of one large hipMemcpyAsync."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    best = 0.0
    with torch.cuda.stream(s):
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            dst.copy_(src, non_blocking=True)
            e1.record(s)
            e1.synchronize()
            best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    return best


def cpu_baseline(shape, T_layer=512):
    """The oracle (fp64 NumPy) on a bounded sample of the same workload: one
    decoder layer forward + backward over 512 tokens, and the head over a
    1/16 slice of the vocabulary; scaled to the full step."""
    from layer_streamed_frozen_amd import store as S
    from layer_streamed_frozen_amd import synth
    from oracle import model as M
    from oracle import nf4 as onf4
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 0) for d in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    W = S.layer_weights_fp32("layer0", shape)
    dense = {}
    for n in S.PROJ:
        p, a = onf4.nf4_quantize(W[n])
        dense[n] = onf4.nf4_dequantize(p, a, W[n].shape).astype(np.float64)
    dense["norm1"] = np.ones(shape.hidden)
    dense["norm2"] = np.ones(shape.hidden)
    ldict = {}  # the same adapter values LoraSet draws for layer 0
    for n, (o, inn) in shape.proj_shapes().items():
        lim = 1.0 / np.sqrt(inn)
        ldict[n] = (synth.uniform(f"lora0.{n}.A", (shape.rank, inn), -lim, lim).astype(np.float64),
                    synth.normal(f"lora0.{n}.B", (o, shape.rank), 0.01).astype(np.float64))
    oc = M.LayerShape(shape.hidden, shape.intermediate, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                      rms_eps=shape.rms_eps, rope_theta=shape.rope_theta, lora_scale=shape.lora_scale)
    x = synth.normal("cpu.x", (1, T_layer, shape.hidden)).astype(np.float64)
    dy = synth.normal("cpu.dy", (1, T_layer, shape.hidden)).astype(np.float64)
    reps, spent = 0, 0.0
    while reps < 2 or (spent < 15.0 and reps < 40):   # about 15 s of CPU work
        t0 = time.perf_counter()
        y, cache = M.layer_fwd(x, dense, ldict, oc)
        M.layer_bwd(dy, dense, ldict, oc, cache)
        spent += time.perf_counter() - t0
        reps += 1
        del y, cache
    t_layer = spent / reps
    V16 = 128256 // 16
    head = synth.normal("cpu.head", (V16, shape.hidden), 0.02).astype(np.float64)
    h = synth.normal("cpu.h", (T_layer, shape.hidden)).astype(np.float64)
    ids = synth.token_ids("cpu.ids", (1, T_layer), V16)
    t0 = time.perf_counter()
    logits = h @ head.T
    lab, val = M.shifted_labels(ids)
    _, dz = M.cross_entropy_fwd_bwd(logits, lab, val)
    _ = dz @ head
    t_head = (time.perf_counter() - t0) * 16
    t_step = 32 * t_layer + t_head
    return {"value": T_layer / t_step, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"one 8B-shaped layer fwd+bwd on {T_layer} tokens, {reps} repetitions averaging "
                       f"{t_layer:.2f} s (x32 layers), plus head fwd+CE+dX on a 1/16 vocabulary slice "
                       f"({t_head / 16:.2f} s, x16); fp64 NumPy"),
            "seconds_measured": round(spent + t_head / 16, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); multi-GPU data-parallel sharding "
              f"is not built in this library.", file=sys.stderr)
        sys.exit(2)
    import torch
    from layer_streamed_frozen_amd import binding as B
    from layer_streamed_frozen_amd import store as S
    from layer_streamed_frozen_amd import synth

    B.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    shape = S.LLAMA8B
    L, V, seq = args.layers, 128256, 512
    batch, accum = {"stack1": (1, 1), "stack4": (4, 4), "dpo": (4, 1), "dpo-unfused": (4, 1)}[args.workload]
    dpo = args.workload.startswith("dpo")
    T = batch * seq

    t0 = time.time()
    log(f"building the NF4 store: {L} layers")
    fmt = {"nf4": B.FMT_NF4, "nf4dq": B.FMT_NF4_DQ, "bf16": B.FMT_BF16}[args.format]
    base_desc = {"nf4": "NF4 base (bs 64, fp32 absmax)", "nf4dq": "NF4 base (bs 64, 8-bit double-quantised absmax)",
                 "bf16": "unquantised bf16 base"}[args.format]

    def weights(i):
        W = S.layer_weights_fp32(f"layer{i}", shape)
        if fmt == B.FMT_BF16:
            for n in S.PROJ:
                W[n] = synth.bf16_exact(W[n])[0].reshape(W[n].shape)
        return W

    store = S.Store(shape, L, fmt=fmt, resident=False, pinned=True, weights_fn=weights)
    log(f"store built in {time.time() - t0:.1f}s: {store.stride * L / 1e9:.3f} GB pinned, "
        f"blob {store.blob_bytes()} B")
    targets = S.PROJ if args.lora_targets == "all" else ("q", "v")
    lora = S.LoraSet(shape, L, targets=targets)
    H = shape.hidden
    emb = torch.from_numpy(synth.bf16_exact(synth.normal("embed", (V, H), 1.0))[1].view(np.int16)) \
        .view(torch.bfloat16).cuda()
    head = torch.from_numpy(synth.bf16_exact(synth.normal("lm_head", (V, H), 0.02))[1].view(np.int16)) \
        .view(torch.bfloat16).cuda()
    fnorm = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    if dpo:
        ids = [torch.from_numpy(synth.preference_pairs("pairs", batch // 2, seq, V, seq // 2)).cuda()]
    else:
        ids = [torch.from_numpy(synth.token_ids(f"ids{m}", (batch, seq), V)).cuda() for m in range(accum)]
    dom = "gate_up_fwd"
    dom_k = B.KERNELS.index(dom)
    # The timed steps carry events around the dominant kernel only; the full
    # per-kernel and copy-engine picture comes from a separate diagnostic pass.
    if args.no_timing:
        flags = 0
    elif args.timing == "all":
        flags = B.STACK_TIMING
    else:
        flags = B.STACK_TIME_KERNEL(dom_k)
    layer_major = accum > 1 and args.accum_order == "layer"
    stack = S.Stack(shape, store, batch, seq, V, flags=flags, keep_activations=args.keep_activations,
                    n_micro=accum if layer_major else 1)
    arr = lora.array()
    opt = (S.AdamW8 if args.optimizer == "adamw8" else S.AdamW)(lora, lr=2e-4)
    torch.cuda.synchronize()

    def step(stk):
        if dpo:
            stk.dpo_step(ids[0], emb, fnorm, head, arr, beta=0.1, fused=args.workload == "dpo",
                         mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
        elif layer_major:
            stk.accum_step(ids, emb, fnorm, head, arr, mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
        else:
            for m in range(accum):
                mode = B.MODE_STREAMED | (B.MODE_ZERO_GRADS if m == 0 else 0)
                stk.step(ids[m], emb, fnorm, head, arr, mode=mode, loss_scale=1.0 / accum)
        opt.step()  # AdamW on every adapter, one launch over the flat arena

    log("measuring the host link")
    link_peak = measure_link_peak(torch)
    log(f"pinned H2D peak {link_peak:.1f} GB/s; warmup {args.warmup}")
    for _ in range(args.warmup):
        step(stack)
    torch.cuda.synchronize()
    B.stack_reset_stats(stack.handle)
    torch.cuda.reset_peak_memory_stats()
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(stack)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st = stack.stats()
    loss = float(stack.loss.item())
    peak_gb = torch.cuda.max_memory_allocated() / 1e9
    tokens = args.steps * accum * T
    value = tokens / elapsed
    ms_step = elapsed / args.steps * 1e3
    log(f"{value:.1f} tok/s, {ms_step:.2f} ms/step, loss {loss:.4f}")

    bytes_step = st.bytes / args.steps
    h2d = {"bytes_per_step": int(bytes_step), "copies_per_step": st.copies / args.steps,
           "GBps_over_step": round(bytes_step / (ms_step * 1e-3) / 1e9, 2),
           "measured_link_peak_GBps": round(link_peak, 2), "pcie5_x16_theoretical_GBps": PCIE5_X16_GBPS}
    flops = gemm_flops(T, shape)
    roof = None
    if st.kernel_launches[dom_k] > 0:
        avg = st.kernel_ms[dom_k] / st.kernel_launches[dom_k] * 1e-3
        ach = flops["gate_up"] / avg / 1e12
        # The counters and the algorithmic bytes belong to the configuration they
        # were taken on: NF4 with fp32 absmax, 512 tokens, recomputing backward.
        measured_cfg = (args.format == "nf4" and T == 512 and not args.keep_activations
                        and args.lora_targets == "all")
        same_src = gemm_src_hash() == GATE_UP_TRAFFIC_SRC
        base = {"nf4": "NF4", "nf4dq": "double-quantised NF4", "bf16": "bf16"}[args.format]
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": round(GATE_UP_TRAFFIC_BYTES) if (same_src and measured_cfg) else None,
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE x1.99975 + WRITE_SIZE x1.000)",
                "algorithmic_bytes": round(GATE_UP_ALGO_BYTES) if measured_cfg else None,
                "kernel": f"fused {base} gate|up GEMM + SwiGLU epilogue, {T}x{2 * shape.intermediate}x{H}",
                "flop_per_launch": flops["gate_up"], "avg_launch_us": round(avg * 1e6, 2),
                "launches": int(st.kernel_launches[dom_k])}

    # diagnostic pass: every kernel class and the copy engine timed with events
    diag_steps = 0 if args.no_timing else args.diag_steps
    dst, delapsed = st, elapsed
    if diag_steps > 0 and flags != B.STACK_TIMING:
        stack.close()
        del stack
        log(f"diagnostic pass: {diag_steps} steps with every kernel and copy timed")
        diag = S.Stack(shape, store, batch, seq, V, flags=B.STACK_TIMING, keep_activations=args.keep_activations,
                       n_micro=accum if layer_major else 1)
        step(diag)
        torch.cuda.synchronize()
        B.stack_reset_stats(diag.handle)
        t1 = time.perf_counter()
        for _ in range(diag_steps):
            step(diag)
        torch.cuda.synchronize()
        delapsed = time.perf_counter() - t1
        dst = diag.stats()
        diag.close()
    else:
        diag_steps = args.steps
        stack.close()
    if dst.copy_ms > 0:
        busy = dst.bytes / (dst.copy_ms * 1e-3) / 1e9
        h2d.update({"GBps_while_copying": round(busy, 2), "frac_of_measured_peak": round(busy / link_peak, 4),
                    "frac_of_theoretical": round(busy / PCIE5_X16_GBPS, 4),
                    "copy_busy_frac_of_step": round(dst.copy_ms / (delapsed * 1e3), 4),
                    "compute_wait_ms_per_step": round(dst.wait_ms / diag_steps, 3),
                    "busy_figures_from": f"diagnostic pass of {diag_steps} steps, "
                                         f"{diag_steps * accum * T / delapsed:.1f} tokens/s with all events on"})
    kernels = {}
    for k, name in enumerate(B.KERNELS):
        n = dst.kernel_launches[k]
        if n == 0:
            continue
        avg_ms = dst.kernel_ms[k] / n
        ent = {"launches_per_step": n / diag_steps, "avg_us": round(avg_ms * 1e3, 2),
               "ms_per_step": round(dst.kernel_ms[k] / diag_steps, 3)}
        base = name.rsplit("_", 1)[0]
        if base in flops:
            tf = flops[base] / (avg_ms * 1e-3) / 1e12
            ent["TFLOPs"] = round(tf, 1)
            ent["mfma_frac"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
        kernels[name] = ent
    gemm_ms = sum(dst.kernel_ms[B.KERNELS.index(n)] for n in B.KERNELS if n.rsplit("_", 1)[0] in flops)
    gemm_flop = sum(flops[n.rsplit("_", 1)[0]] * dst.kernel_launches[B.KERNELS.index(n)]
                    for n in B.KERNELS if n.rsplit("_", 1)[0] in flops)
    layer_gemms = None
    if gemm_ms > 0:
        tf = gemm_flop / (gemm_ms * 1e-3) / 1e12
        layer_gemms = {"TFLOPs": round(tf, 1), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                       "ms_per_step": round(gemm_ms / diag_steps, 2)}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded random weights and token ids)",
        "config": {"workload": (f"streamed {L}-layer Llama-3.1-8B-shaped stack, {base_desc}, "
                                f"LoRA r16 on {','.join(targets)}, vocab {V}, "
                                + (f"DPO beta 0.1 over {batch // 2} chosen/rejected pairs x seq {seq}, "
                                   f"reference = adapters off, "
                                   + ("fused into the policy's layer visit" if args.workload == "dpo"
                                      else "separate reference pass") if dpo else
                                   f"batch {batch} x seq {seq}, accumulation {accum}"
                                   + ((", one walk over the stack per direction for all micro-batches"
                                       if layer_major else ", the stack walked once per micro-batch")
                                      if accum > 1 else ""))),
                   "global_batch": batch * accum, "seq_len": seq, "layers": L, "vocab": V,
                   "optimizer": ("AdamW lr 2e-4, fp32 moments, once per step" if args.optimizer == "adamw" else
                                 "AdamW lr 2e-4, 8-bit block-wise moments (blocks of 2048, dynamic code), "
                                 "once per step"),
                   "backward": ("forward intermediates kept in HBM, no recompute" if args.keep_activations
                                else "per-layer recompute from the checkpoint"),
                   "parallelism": "single GPU"},
        "h2d": h2d, "roofline": roof, "layer_gemms": layer_gemms, "kernels": kernels,
        "peak_device_GB": round(peak_gb, 3),
        "loss": loss,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(shape)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
