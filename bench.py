"""Throughput of the streamed NF4 + LoRA training step on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--repeat 3]
                    [--workload stack1|stack4|stack16|dpo|dpo-unfused|layer|linear]
                    [--format nf4|nf4dq|bf16] [--optimizer adamw|adamw8] [--lora-targets all|qv]
                    [--accum-order layer|micro] [--keep-activations] [--no-cpu-baseline] [--no-extra]
                    [--one-copy-stream]

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
the stack once per micro-batch instead; both give the same bits).  "stack16" is the
same 16 sequences of 512 as one batch of 8192 tokens (no accumulation).  "dpo" is the preference-loss step: 2
chosen/rejected pairs of 512 tokens (4 sequences, pair p sharing a 256-token
prompt), DPO with beta 0.1, the reference log-probabilities from the same
streamed base with the adapters off, computed in the policy's layer visit
("dpo-unfused": in a separate pass over the stack).  "layer" is one 8B-shaped
decoder layer at 512 tokens, resident: forward, then the backward that
recomputes it (t_fwd, t_bwd, layer tokens/s, per-kernel MFMA fractions).
"linear" is one 256 x 256 NF4 linear with a rank-8 LoRA adapter over 64
tokens, forward + backward (latency; launch-bound, no roofline claim).  Inputs
and weights are seeded synthetic data.

Prints one JSON line.  ``value`` is tokens per second over the timed steps,
with every input already resident (the frozen store in pinned host memory is
the method's input; its per-step host-to-device traffic is part of the step).
The timed steps carry HIP events around the gate|up forward GEMM only (the
``roofline`` kernel); a diagnostic pass of a few more steps afterwards times
every kernel class and every copy (``kernels``, ``layer_gemms`` and the
copy-engine figures in ``h2d``), since events on every kernel and copy slow
the step by a few percent.  The timed region runs ``--repeat`` times (each
``--steps`` steps); ``value`` is the mean, and ``repeat`` lists every run with
the standard deviation.  With every option at its default, the same run then
times a few steps of "stack4" and "dpo" on the same store (``other_workloads``;
``--no-extra`` skips them).
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
# (profiles/pmc_traffic_layer8b_seq512.md): FETCH_SIZE 50043.05 KiB scaled by 1.99975
# (the calibration kernel's ratio) + WRITE_SIZE 28737.24 KiB scaled by 1.0.  Valid only
# for the sources of that kernel they were taken on (hash below); otherwise null.
GATE_UP_TRAFFIC_BYTES = (50043.05 * 1.99975 + 28737.24 * 1.0) * 1024
GATE_UP_TRAFFIC_SRC = "895059a4b4dea2d0"
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
    p.add_argument("--repeat", type=int, default=3, help="timed runs of --steps steps each (mean and sd)")
    p.add_argument("--workload", choices=["stack1", "stack4", "stack16", "dpo", "dpo-unfused", "layer", "linear"],
                   default="stack1")
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--tokens", type=int, default=512,
                   help="layer workload: tokens per call (sequences of 512)")
    p.add_argument("--wide-tile", type=int, choices=[0, 1, 256, 512], default=1,
                   help="diagnostics: kernel of the wide forward GEMMs (1: by shape, 256/512: that tile's rows, "
                        "0: the general kernel); every choice gives the same bits")
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
    p.add_argument("--one-copy-stream", action="store_true",
                   help="copy each layer as one transfer on one copy stream (default: two halves on two)")
    p.add_argument("--no-extra", action="store_true",
                   help="stack1 with the defaults also times the stack4 and fused-DPO steps on the same store "
                        "(a few steps each, in the same run); this skips them")
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
    """Best pinned host -> device copy rate (GB/s) of one large hipMemcpyAsync,
    on the copy stream the stacks use (no extra stream for HIP to place)."""
    from layer_streamed_frozen_amd.store import copy_stream
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = copy_stream()
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


def host_info():
    """The CPU the oracle baseline runs on: core counts, the BLAS threads NumPy
    uses, and the model name."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([d.get("num_threads", 0) for d in threadpool_info()] + [0]) or None
    except Exception:
        blas = None
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "blas_threads": blas,
            "cpu_model": model}


def _link_gbps(speed, width):
    """Theoretical one-direction PCIe rate from sysfs strings ("32.0 GT/s PCIe", "16")."""
    try:
        gts = float(speed.split()[0])
        lanes = int(width)
    except (ValueError, IndexError, AttributeError):
        return None
    enc = 128.0 / 130.0 if gts >= 8.0 else 0.8
    return round(gts * lanes * enc / 8.0, 2)


def pcie_link(torch):
    """The GPU's PCIe link as sysfs reports it: the device's own link and the
    upstream ports between it and the root complex (speed, width, theoretical
    GB/s)."""
    props = torch.cuda.get_device_properties(0)
    dom, bus, dev = (getattr(props, k, None) for k in ("pci_domain_id", "pci_bus_id", "pci_device_id"))
    path = None
    if bus is not None and dev is not None:
        cand = f"/sys/bus/pci/devices/{(dom or 0):04x}:{bus:02x}:{dev:02x}.0"
        if os.path.exists(cand):
            path = cand
    if path is None:
        return {"found": False}
    out = {"found": True, "bdf": os.path.basename(path), "hops": []}
    p = os.path.realpath(path)
    while os.path.basename(p).count(":") == 2:
        def rd(name):
            try:
                with open(os.path.join(p, name)) as f:
                    return f.read().strip()
            except OSError:
                return None
        cs, cw, ms, mw = rd("current_link_speed"), rd("current_link_width"), rd("max_link_speed"), rd("max_link_width")
        if cs is not None:
            out["hops"].append({"bdf": os.path.basename(p), "current_speed": cs, "current_width": cw,
                                "max_speed": ms, "max_width": mw, "current_GBps": _link_gbps(cs, cw)})
        p = os.path.dirname(p)
    if out["hops"]:
        rates = [h["current_GBps"] for h in out["hops"] if h["current_GBps"]]
        out["narrowest_GBps"] = min(rates) if rates else None
    return out


def _oracle_layer(shape, prefix, dtype):
    """Dense oracle weights (the oracle's own NF4 round trip) and the adapters
    LoraSet draws for layer 0, in dtype."""
    from layer_streamed_frozen_amd import store as S
    from layer_streamed_frozen_amd import synth
    from oracle import nf4 as onf4
    W = S.layer_weights_fp32(prefix, shape)
    dense = {}
    for n in S.PROJ:
        p, a = onf4.nf4_quantize(W[n])
        dense[n] = onf4.nf4_dequantize(p, a, W[n].shape).astype(dtype)
    dense["norm1"] = np.ones(shape.hidden, dtype)
    dense["norm2"] = np.ones(shape.hidden, dtype)
    ldict = {}
    for n, (o, inn) in shape.proj_shapes().items():
        lim = 1.0 / np.sqrt(inn)
        ldict[n] = (synth.uniform(f"lora0.{n}.A", (shape.rank, inn), -lim, lim).astype(dtype),
                    synth.normal(f"lora0.{n}.B", (o, shape.rank), 0.01).astype(dtype))
    return dense, ldict


def cpu_baseline(shape, workload, T_layer=512, budget_s=15.0):
    """The oracle (NumPy, fp32 arrays, multithreaded BLAS) on a bounded sample
    of the workload, on this host's cores: one decoder layer forward + backward
    over 512 tokens (repeated for about budget_s), and for the stack workloads
    also the head over a 1/16 slice of the vocabulary; scaled to the unit of
    the GPU line."""
    from layer_streamed_frozen_amd import synth
    from oracle import model as M
    from oracle import nf4 as onf4
    dt = np.float32
    info = host_info()
    cores = info["blas_threads"] or info["affinity_cpus"]
    if workload == "linear":
        W = synth.normal("cfg1.W", (256, 256), 0.02)
        p, a = onf4.nf4_quantize(W)
        Wd = onf4.nf4_dequantize(p, a, W.shape).astype(dt)
        A = synth.uniform("cfg1.A", (8, 256), -1 / 16, 1 / 16).astype(dt)
        Bm = synth.normal("cfg1.B", (256, 8), 0.01).astype(dt)
        x = synth.bf16_exact(synth.normal("cfg1.X", (64, 256)))[0].astype(dt)
        dy = synth.bf16_exact(synth.normal("cfg1.dY", (64, 256)))[0].astype(dt)
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(budget_s, 5.0):
            y, u = M.lora_linear_fwd(x, Wd, A, Bm, 2.0)
            M.lora_linear_bwd(dy, x, Wd, A, Bm, 2.0, u)
            reps += 1
        spent = time.perf_counter() - t0
        return {"value": round(spent / reps * 1e6, 2), "unit": "us per fwd+bwd", "cores": int(cores),
                "kind": "oracle", "dtype": "fp32", "host": info,
                "sample": f"the same 256x256 NF4 linear + rank-8 LoRA over 64 tokens, {reps} fwd+bwd repetitions",
                "seconds_measured": round(spent, 2)}
    dense, ldict = _oracle_layer(shape, "layer0", dt)
    oc = M.LayerShape(shape.hidden, shape.intermediate, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                      rms_eps=shape.rms_eps, rope_theta=shape.rope_theta, lora_scale=shape.lora_scale)
    x = synth.normal("cpu.x", (1, T_layer, shape.hidden)).astype(dt)
    dy = synth.normal("cpu.dy", (1, T_layer, shape.hidden)).astype(dt)
    reps, spent = 0, 0.0
    while reps < 2 or (spent < budget_s and reps < 40):
        t0 = time.perf_counter()
        y, cache = M.layer_fwd(x, dense, ldict, oc)
        M.layer_bwd(dy, dense, ldict, oc, cache)
        spent += time.perf_counter() - t0
        reps += 1
        del y, cache
    t_layer = spent / reps
    if workload == "layer":
        return {"value": round(T_layer / t_layer, 2), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
                "dtype": "fp32", "host": info,
                "sample": (f"one 8B-shaped layer forward + backward on {T_layer} tokens, {reps} repetitions "
                           f"averaging {t_layer:.2f} s"),
                "seconds_measured": round(spent, 2)}
    V16 = 128256 // 16
    head = synth.normal("cpu.head", (V16, shape.hidden), 0.02).astype(dt)
    h = synth.normal("cpu.h", (T_layer, shape.hidden)).astype(dt)
    ids = synth.token_ids("cpu.ids", (1, T_layer), V16)
    t0 = time.perf_counter()
    logits = h @ head.T
    lab, val = M.shifted_labels(ids)
    _, dz = M.cross_entropy_fwd_bwd(logits, lab, val)
    _ = dz.astype(dt) @ head
    t_head = (time.perf_counter() - t0) * 16
    t_step = 32 * t_layer + t_head
    return {"value": round(T_layer / t_step, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "dtype": "fp32", "host": info,
            "sample": (f"one 8B-shaped layer fwd+bwd on {T_layer} tokens, {reps} repetitions averaging "
                       f"{t_layer:.2f} s (x32 layers), plus head fwd+CE+dX on a 1/16 vocabulary slice "
                       f"({t_head / 16:.2f} s, x16); per-token rate of a 512-token step"),
            "seconds_measured": round(spent + t_head / 16, 2)}


def mean_sd(v):
    a = np.asarray(v, dtype=np.float64)
    return float(a.mean()), float(a.std(ddof=1)) if len(a) > 1 else 0.0


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
    if args.wide_tile != 1:
        B.gemm_set_wide(args.wide_tile if args.wide_tile else False)
    shape = S.LLAMA8B
    if args.workload in ("linear", "layer"):
        out = (run_linear if args.workload == "linear" else run_layer)(args, torch, B, S, synth)
        out["pcie_link"] = pcie_link(torch)
        if not args.no_cpu_baseline:
            log("timing the CPU oracle on a bounded sample")
            out["cpu_baseline"] = cpu_baseline(shape, args.workload)
        print(json.dumps(out), flush=True)
        return
    L, V, seq = args.layers, 128256, 512
    batch, accum = {"stack1": (1, 1), "stack4": (4, 4), "stack16": (16, 1), "dpo": (4, 1),
                    "dpo-unfused": (4, 1)}[args.workload]
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
    copy_flags = B.STACK_ONE_COPY_STREAM if args.one_copy_stream else 0
    flags |= copy_flags
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
    runs = []
    for r in range(max(1, args.repeat)):
        log(f"timing {args.steps} steps (run {r + 1} of {max(1, args.repeat)})")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(stack)
        torch.cuda.synchronize()
        runs.append(time.perf_counter() - t0)
    n_timed = args.steps * len(runs)
    elapsed = sum(runs)
    st = stack.stats()
    loss = float(stack.loss.item())
    peak_gb = torch.cuda.max_memory_allocated() / 1e9
    tokens = args.steps * accum * T
    rates = [tokens / e for e in runs]
    value, value_sd = mean_sd(rates)
    ms_step = elapsed / n_timed * 1e3
    log(f"{value:.1f} +- {value_sd:.1f} tok/s over {len(runs)} runs, {ms_step:.2f} ms/step, loss {loss:.4f}")

    bytes_step = st.bytes / n_timed
    h2d = {"copy_streams": 1 if args.one_copy_stream else 2,
           "bytes_per_step": int(bytes_step), "copies_per_step": st.copies / n_timed,
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
        diag = S.Stack(shape, store, batch, seq, V, flags=B.STACK_TIMING | copy_flags,
                       keep_activations=args.keep_activations,
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
                                         f"{diag_steps * accum * T / delapsed:.1f} tokens/s with all events on"
                                         + ("" if args.one_copy_stream else
                                            "; per-copy timing forks and joins the two copy streams per layer "
                                            "(one event pair per layer copy), the timed steps do not")})
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
    # With micro-batches on two streams (accumulation in one walk, recomputing
    # backward) a launch's event pair also spans the other stream's kernels, so
    # the roofline kernel is timed in the diagnostic pass, which runs them on
    # one stream.
    two_streams = layer_major and not args.keep_activations
    if roof is not None and two_streams and dst is not st and dst.kernel_launches[dom_k] > 0:
        avg = dst.kernel_ms[dom_k] / dst.kernel_launches[dom_k] * 1e-3
        ach = flops["gate_up"] / avg / 1e12
        roof.update({"achieved": round(ach, 1), "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                     "avg_launch_us": round(avg * 1e6, 2), "launches": int(dst.kernel_launches[dom_k]),
                     "timed_in": "diagnostic pass (micro-batches on one stream; the timed steps run two "
                                 "micro-batches at a time on two streams)"})
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
        "repeat": {"n": len(runs), "tokens_per_s": [round(v, 2) for v in rates], "mean": round(value, 2),
                   "sd": round(value_sd, 2)},
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
        "h2d": h2d, "pcie_link": pcie_link(torch), "roofline": roof, "layer_gemms": layer_gemms,
        "kernels": kernels,
        "peak_device_GB": round(peak_gb, 3),
        "loss": loss,
    }
    default_cfg = (args.workload == "stack1" and args.format == "nf4" and args.lora_targets == "all"
                   and args.optimizer == "adamw" and not args.keep_activations and L == 32
                   and not args.one_copy_stream)
    if default_cfg and not args.no_extra:
        out["other_workloads"] = other_workloads(torch, B, S, synth, shape, store, lora, arr, opt, emb, fnorm,
                                                 head, V, seq)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(shape, args.workload)
    print(json.dumps(out), flush=True)


def other_workloads(torch, B, S, synth, shape, store, lora, arr, opt, emb, fnorm, head, V, seq, warmup=1, steps=3,
                    repeat=2):
    """The compute-bound steps on the store the headline was measured on, a
    few steps each (the same step code as --workload stack4 and --workload
    dpo, without per-kernel events): 4 micro-batches of 4 x 512 tokens served
    by one walk over the stack per direction, and DPO over 2 chosen/rejected
    pairs x 512 with the reference pass fused into the policy's layer visit.
    Each step ends with one AdamW update."""
    res = {}
    for kind in ("stack4", "dpo"):
        batch, accum = (4, 4) if kind == "stack4" else (4, 1)
        if kind == "dpo":
            ids = [torch.from_numpy(synth.preference_pairs("pairs", batch // 2, seq, V, seq // 2)).cuda()]
        else:
            ids = [torch.from_numpy(synth.token_ids(f"ids{m}", (batch, seq), V)).cuda() for m in range(accum)]
        stk = S.Stack(shape, store, batch, seq, V, flags=0, n_micro=accum if kind == "stack4" else 1)

        def one():
            if kind == "dpo":
                stk.dpo_step(ids[0], emb, fnorm, head, arr, beta=0.1, fused=True,
                             mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
            else:
                stk.accum_step(ids, emb, fnorm, head, arr, mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
            opt.step()

        log(f"other workload {kind}: {warmup} warm-up + {repeat} x {steps} steps")
        for _ in range(warmup):
            one()
        torch.cuda.synchronize()
        B.stack_reset_stats(stk.handle)
        runs = []
        for _ in range(repeat):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                one()
            torch.cuda.synchronize()
            runs.append(time.perf_counter() - t0)
        st = stk.stats()
        stk.close()
        tokens = steps * accum * batch * seq
        rates = [tokens / e for e in runs]
        v, sd = mean_sd(rates)
        n = steps * len(runs)
        res[kind] = {"tokens_per_s": round(v, 2), "sd": round(sd, 2), "runs": len(runs), "steps": steps,
                     "warmup": warmup, "ms_per_step": round(sum(runs) / n * 1e3, 3),
                     "copies_per_step": st.copies / n,
                     "GBps_over_step": round(st.bytes / n / (sum(runs) / n) / 1e9, 2),
                     "workload": ("batch 4 x seq 512, accumulation 4, one walk over the stack per direction "
                                  "for all micro-batches" if kind == "stack4" else
                                  "DPO beta 0.1, 2 chosen/rejected pairs x seq 512, reference = adapters off, "
                                  "fused into the policy's layer visit")}
        log(f"other workload {kind}: {v:.1f} +- {sd:.1f} tok/s")
    return res


def _events(torch, fn, n):
    """Average ms of fn() over n calls, by events on the current stream."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(n):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / n


def run_linear(args, torch, B, S, synth):
    """One 256 x 256 NF4 linear + rank-8 LoRA (alpha 16) over 64 tokens:
    forward + backward latency."""
    n_out = n_in = 256
    T, r, scale = 64, 8, 2.0
    W = synth.normal("cfg1.W", (n_out, n_in), 0.02)
    packed, absmax = B.nf4_quantize(torch.from_numpy(W.reshape(-1)).cuda())
    w = B.weight(packed, absmax)
    A = torch.from_numpy(synth.uniform("cfg1.A", (r, n_in), -1 / 16, 1 / 16)).cuda()
    Bm = torch.from_numpy(synth.normal("cfg1.B", (n_out, r), 0.01)).cuda()
    bits = lambda name, shp: torch.from_numpy(synth.bf16_exact(synth.normal(name, shp))[1].view(np.int16)) \
        .view(torch.bfloat16).cuda()
    x, dy = bits("cfg1.X", (T, n_in)), bits("cfg1.dY", (T, n_out))
    ws = torch.empty(B.linear_workspace_bytes(T, n_out, n_in, r), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, n_out), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((T, n_in), dtype=torch.bfloat16, device="cuda")
    dA = torch.zeros((r, n_in), dtype=torch.float32, device="cuda")
    dB = torch.zeros((n_out, r), dtype=torch.float32, device="cuda")
    fwd = lambda: B.linear_fwd(w, B.FMT_NF4, n_out, n_in, A, Bm, r, scale, x, y, ws)
    bwd = lambda: B.linear_bwd(w, B.FMT_NF4, n_out, n_in, A, Bm, r, scale, x, dy, dx, dA, dB, ws)
    both = lambda: (fwd(), bwd())
    for _ in range(args.warmup):
        both()
    torch.cuda.synchronize()
    steps = max(args.steps, 200)
    runs = [_events(torch, both, steps) * 1e3 for _ in range(max(1, args.repeat))]
    t_f = _events(torch, fwd, steps) * 1e3
    t_b = _events(torch, bwd, steps) * 1e3
    value, sd = mean_sd(runs)
    log(f"linear fwd+bwd {value:.2f} +- {sd:.2f} us (fwd {t_f:.2f}, bwd {t_b:.2f})")
    return {"metric": "single NF4 linear + LoRA fwd+bwd latency (256x256, r 8, 64 tokens)", "value": round(value, 2),
            "unit": "us", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
            "repeat": {"n": len(runs), "us": [round(v, 2) for v in runs], "mean": round(value, 2),
                       "sd": round(sd, 2)},
            "ms_per_step": round(value / 1e3, 5), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic (seeded)",
            "config": {"workload": "one 256x256 NF4 linear (bs 64, fp32 absmax) + LoRA r 8 alpha 16, 64 tokens, "
                                   "forward + backward (dx, dA, dB)", "parallelism": "single GPU"},
            "t_fwd_us": round(t_f, 2), "t_bwd_us": round(t_b, 2),
            "roofline": None, "roofline_note": "launch-bound (a few microseconds of kernels); no roofline claim"}


def run_layer(args, torch, B, S, synth):
    """One 8B-shaped NF4 decoder layer (LoRA r16 on all seven projections) at
    512 tokens, resident: forward, then the recomputing backward."""
    shape = S.LLAMA8B
    T, H = args.tokens, shape.hidden
    if T % 512:
        raise SystemExit("--tokens must be a multiple of 512")
    W = S.layer_weights_fp32("layer0", shape)
    blob = S.build_layer_blob(shape, W)
    cfg = shape.cfg(T // 512, 512)
    lw = B.layer_weights_from_blob(cfg, B.FMT_NF4, blob.data_ptr())
    lora = S.LoraSet(shape, 1)
    bits = lambda name: torch.from_numpy(synth.bf16_exact(synth.normal(name, (T, H)))[1].view(np.int16)) \
        .view(torch.bfloat16).cuda()
    x, dy = bits("layer.x"), bits("layer.dy")
    ws = torch.empty(B.layer_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    y, dx = torch.empty_like(x), torch.empty_like(x)
    ls = lora.struct(0)
    fwd = lambda: B.layer_fwd(cfg, lw, ls, x, y, ws)
    bwd = lambda: B.layer_bwd(cfg, lw, ls, x, dy, dx, ws)
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    steps = max(args.steps, 10)
    t_f, t_b, rates = [], [], []
    for _ in range(max(1, args.repeat)):
        f = _events(torch, fwd, steps)
        b = _events(torch, bwd, steps)
        t_f.append(f)
        t_b.append(b)
        rates.append(T / ((f + b) * 1e-3))
    value, sd = mean_sd(rates)
    tf, tb = float(np.mean(t_f)), float(np.mean(t_b))
    log(f"layer: fwd {tf:.3f} ms, bwd {tb:.3f} ms, {value:.1f} +- {sd:.1f} tok/s")
    # per-kernel classes: the same layer as a one-layer resident stack with every kernel timed
    store = S.Store(shape, 1, resident=True, pinned=True, weights_fn=lambda i: W)
    V = 1024
    stack = S.Stack(shape, store, T // 512, 512, V, flags=B.STACK_TIMING)
    emb = torch.from_numpy(synth.bf16_exact(synth.normal("layer.embed", (V, H), 1.0))[1].view(np.int16)) \
        .view(torch.bfloat16).cuda()
    head = torch.from_numpy(synth.bf16_exact(synth.normal("layer.head", (V, H), 0.02))[1].view(np.int16)) \
        .view(torch.bfloat16).cuda()
    fnorm = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    ids = torch.from_numpy(synth.token_ids("layer.ids", (T // 512, 512), V)).cuda()
    arr = lora.array()
    stack.step(ids, emb, fnorm, head, arr, mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    torch.cuda.synchronize()
    B.stack_reset_stats(stack.handle)
    n_diag = max(1, args.diag_steps)
    for _ in range(n_diag):
        stack.step(ids, emb, fnorm, head, arr, mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    torch.cuda.synchronize()
    st = stack.stats()
    stack.close()
    flops = gemm_flops(T, shape)
    kernels, gemm_ms, gemm_flop = {}, 0.0, 0.0
    for k, name in enumerate(B.KERNELS):
        n = st.kernel_launches[k]
        base = name.rsplit("_", 1)[0]
        if n == 0 or base not in flops:
            continue
        avg_ms = st.kernel_ms[k] / n
        tf_s = flops[base] / (avg_ms * 1e-3) / 1e12
        kernels[name] = {"launches_per_layer_pass": n / n_diag, "avg_us": round(avg_ms * 1e3, 2),
                         "TFLOPs": round(tf_s, 1), "mfma_frac": round(tf_s / MFMA_BF16_PEAK_TFLOPS, 4)}
        gemm_ms += st.kernel_ms[k]
        gemm_flop += flops[base] * n
    layer_gemms = None
    if gemm_ms > 0:
        tfl = gemm_flop / (gemm_ms * 1e-3) / 1e12
        layer_gemms = {"TFLOPs": round(tfl, 1), "mfma_frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
                       "ms_per_layer_pass": round(gemm_ms / n_diag, 3)}
    dom = kernels.get("gate_up_fwd")
    roof = None
    if dom:
        roof = {"bound": "mfma", "achieved": dom["TFLOPs"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": dom["mfma_frac"], "traffic": None,
                "kernel": f"fused NF4 gate|up GEMM + SwiGLU epilogue, {T}x{2 * shape.intermediate}x{H}",
                "avg_launch_us": dom["avg_us"]}
    return {"metric": "one 8B-shape NF4+LoRA decoder layer fwd + recompute-bwd, tokens/s", "value": round(value, 2),
            "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
            "repeat": {"n": len(rates), "tokens_per_s": [round(v, 2) for v in rates], "mean": round(value, 2),
                       "sd": round(sd, 2)},
            "ms_per_step": round(tf + tb, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic (seeded random weights and activations)",
            "config": {"workload": "one Llama-3.1-8B-shaped decoder layer, NF4 base (bs 64, fp32 absmax), LoRA r16 on "
                                   f"q,k,v,o,gate,up,down, batch {T // 512} x seq 512, resident, forward + recomputing "
                                   "backward", "parallelism": "single GPU"},
            "t_fwd_ms": round(tf, 4), "t_bwd_ms": round(tb, 4),
            "roofline": roof, "layer_gemms": layer_gemms, "kernels": kernels,
            "kernels_from": f"the same layer as a one-layer resident stack, {n_diag} steps with every kernel timed"}


if __name__ == "__main__":
    main()
