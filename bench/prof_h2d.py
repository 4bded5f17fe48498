"""Host-to-device rate of one 8B-shaped NF4 layer blob (122,699,776 bytes)
copied on its own: from a pinned store of --layers such blobs into one of two
device buffers, one hipMemcpyAsync per copy, with and without a bf16 GEMM load
on another stream, and the same copy cut in two on two streams.

    python3 bench/prof_h2d.py [--layers 32] [--reps 64] [--sustain SECONDS [--idle]] [--probe-gaps]
                              [--step-pattern [--pieces N]]

Prints, per variant, the median, minimum and maximum copy time (event-timed).
With --sustain, instead copies back to back for about that long while bf16
GEMMs keep another stream busy, without synchronising in between (as in the
streamed step), and prints the median copy time of each tenth of the run;
--idle leaves the GPU without other work.  With --probe-gaps, instead times
runs of 24 back-to-back copies on one stream (the average per copy, so any idle
time between copies counts): plain; each followed by an event record; each
preceded by a wait on an event of another stream that completed long before;
each preceded by a wait on an event recorded on another stream just before;
then 64 copies cycling over 8 and over all --layers blobs of the store, in
order and in a stride-7 order.  With --step-pattern, replays the streamed
512-token step's schedule outside the library's stack: a forward walk over the
32 layers (this library's layer_fwd of one 8B-shaped NF4 layer), the two
lm_head GEMMs of the head, a backward walk (layer_bwd, recomputing), and an
optimizer-sized HBM pass, the layer copies on their own stream ordered by
events exactly as the streamer does (two device buffers, the last two layers
of a walk reused by the next), and prints every copy's duration for three
steps and the per-step time over ten; --pieces N sends each layer as N equal
pieces (4 KiB multiples) on N copy streams that fork from and join back into
the first, as the library's stack does with two.
"""
import argparse
import statistics

import torch

BLOB = 122699776


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--reps", type=int, default=64)
    ap.add_argument("--sustain", type=float, default=0.0)
    ap.add_argument("--idle", action="store_true")
    ap.add_argument("--probe-gaps", action="store_true")
    ap.add_argument("--step-pattern", action="store_true")
    ap.add_argument("--pieces", type=int, default=1)
    args = ap.parse_args()
    nl = args.layers
    if args.step_pattern:
        step_pattern(torch, nl, args.pieces)
        return
    src = torch.empty(nl * BLOB, dtype=torch.uint8, pin_memory=True)
    src.fill_(1)
    dst = [torch.empty(BLOB, dtype=torch.uint8, device="cuda") for _ in range(2)]
    s1, s2, sc = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    a = torch.randn(4096, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)

    def load(n):
        with torch.cuda.stream(sc):
            for _ in range(n):
                torch.mm(a, b)

    def run(pieces, busy):
        ts = []
        for r in range(args.reps):
            j = r % nl
            sv = src[j * BLOB:(j + 1) * BLOB]
            d = dst[r % 2]
            if busy:
                load(6)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s1)
            if pieces == 1:
                with torch.cuda.stream(s1):
                    d.copy_(sv, non_blocking=True)
            else:
                ev = torch.cuda.Event()
                ev.record(s1)
                s2.wait_event(ev)
                h = (BLOB // 2) // 4096 * 4096
                with torch.cuda.stream(s1):
                    d[:h].copy_(sv[:h], non_blocking=True)
                with torch.cuda.stream(s2):
                    d[h:].copy_(sv[h:], non_blocking=True)
                ev2 = torch.cuda.Event()
                ev2.record(s2)
                s1.wait_event(ev2)
            e1.record(s1)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return ts

    if args.probe_gaps:
        probe_gaps(torch, src, dst, s1, s2, nl)
        return

    if args.sustain > 0:
        n = max(20, int(args.sustain * 1e6 / 2200))
        evs = []
        for r in range(n):
            j = r % nl
            if not args.idle:
                load(4)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s1)
            with torch.cuda.stream(s1):
                dst[r % 2].copy_(src[j * BLOB:(j + 1) * BLOB], non_blocking=True)
            e1.record(s1)
            evs.append((e0, e1))
            if r % 64 == 63:  # keep the host at most a few hundred copies ahead
                evs[r - 32][1].synchronize()
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) * 1e3 for a, b in evs]
        k = max(1, n // 10)
        for i in range(0, n - k + 1, k):
            blk = ts[i:i + k]
            slow = sum(1 for t in blk if t > 2300)
            print(f"[prof_h2d] sustained copies{' (idle GPU)' if args.idle else ''} {i}..{i + k - 1}: "
                  f"median {statistics.median(blk):.0f} us, mean {statistics.mean(blk):.0f}, max {max(blk):.0f}, "
                  f"over 2.3 ms {slow}/{len(blk)}", flush=True)
        return

    for busy in (False, True):
        for pieces in (1, 2):
            run(pieces, busy)  # warm
            ts = run(pieces, busy)
            med = statistics.median(ts)
            print(f"[prof_h2d] GEMM load on another stream: {busy}, streams: {pieces}: median {med:.0f} us "
                  f"({BLOB / med / 1e3:.2f} GB/s), min {min(ts):.0f}, max {max(ts):.0f}", flush=True)


def step_pattern(torch, L, pieces=1):
    import os
    import sys
    import numpy as np
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from layer_streamed_frozen_amd import binding as B
    from layer_streamed_frozen_amd import store as S
    from layer_streamed_frozen_amd import synth
    B.lib()
    shape = S.LLAMA8B
    W = S.layer_weights_fp32("h2d.layer", shape)
    blob = S.build_layer_blob(shape, W)
    cfg = shape.cfg(1, 512)
    H, V = shape.hidden, 128256
    lora = S.LoraSet(shape, 1, prefix="h2d.lora")

    def bf16_in(name):
        return torch.from_numpy(synth.bf16_exact(synth.normal(name, (512, H)))[1].view(np.int16)) \
            .view(torch.bfloat16).cuda()

    x, dy = bf16_in("h2d.x"), bf16_in("h2d.dy")
    ws = torch.empty(B.layer_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    y, dx = torch.empty_like(x), torch.empty_like(x)
    ls = lora.struct(0)
    src = torch.empty(L * BLOB, dtype=torch.uint8, pin_memory=True)
    hb = blob.cpu()
    for j in range(L):  # every layer the same bytes: only the copies' timing matters here
        src[j * BLOB:(j + 1) * BLOB].copy_(hb[:BLOB])
    dst = [torch.empty(BLOB, dtype=torch.uint8, device="cuda") for _ in range(2)]
    lws = [B.layer_weights_from_blob(cfg, B.FMT_NF4, d.data_ptr()) for d in dst]
    head = torch.randn(V, H, device="cuda", dtype=torch.bfloat16) * 0.02
    opt_buf = torch.empty(1170 * 1000 * 1000 // 4, dtype=torch.float32, device="cuda")
    cs, cp = torch.cuda.current_stream(), torch.cuda.Stream()
    extra = [torch.cuda.Stream() for _ in range(pieces - 1)]
    cut = [0] + [BLOB // pieces // 4096 * 4096 * k for k in range(1, pieces)] + [BLOB]
    slot, ready, freed, cev = [None, None], [None, None], [None, None], []

    def acquire(j, b):
        if slot[b] == j:
            return
        if freed[b] is not None:
            cp.wait_event(freed[b])
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(cp)
        for s in extra:
            s.wait_event(e0)
        for k, s in enumerate([cp] + extra):
            with torch.cuda.stream(s):
                dst[b][cut[k]:cut[k + 1]].copy_(src[j * BLOB + cut[k]:j * BLOB + cut[k + 1]], non_blocking=True)
        for s in extra:
            done = torch.cuda.Event()
            done.record(s)
            cp.wait_event(done)
        e1.record(cp)
        cev.append((e0, e1))
        ready[b] = torch.cuda.Event()
        ready[b].record(cp)
        slot[b] = j

    def walk(forward):
        order = list(range(L)) if forward else list(range(L - 1, -1, -1))
        acquire(order[0], order[0] & 1)
        acquire(order[1], order[1] & 1)
        for n, j in enumerate(order):
            b = j & 1
            cs.wait_event(ready[b])
            if forward:
                B.layer_fwd(cfg, lws[b], ls, x, y, ws, stream=cs)
            else:
                B.layer_bwd(cfg, lws[b], ls, x, dy, dx, ws, stream=cs)
            freed[b] = torch.cuda.Event()
            freed[b].record(cs)
            if n + 2 < L:
                acquire(order[n + 2], b)

    def step():
        walk(True)
        logits = x @ head.t()
        _ = logits @ head
        walk(False)
        opt_buf.mul_(0.999)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    cev.clear()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    n_steps = 10
    t0.record(cs)
    for _ in range(n_steps):
        step()
    t1.record(cs)
    torch.cuda.synchronize()
    d = [a.elapsed_time(b) * 1e3 for a, b in cev]
    per = len(d) // n_steps
    for k in range(3):
        print(f"[prof_h2d] step pattern, copy durations of step {k} (ms): "
              + " ".join(f"{v / 1000:.2f}" for v in d[k * per:(k + 1) * per]), flush=True)
    total = t0.elapsed_time(t1)
    print(f"[prof_h2d] step pattern, {pieces} piece(s) per copy: {total / n_steps:.2f} ms per step, {per} copies "
          f"per step, copy median "
          f"{statistics.median(d):.0f} us, mean {statistics.mean(d):.0f} us, copy engine busy "
          f"{sum(d) / 1e3 / total:.3f} of the time", flush=True)


def probe_gaps(torch, src, dst, s1, s2, nl):
    def timed(n, body):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s1)
        for r in range(n):
            body(r)
        e1.record(s1)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    def copy(r, j):
        with torch.cuda.stream(s1):
            dst[r % 2].copy_(src[j * BLOB:(j + 1) * BLOB], non_blocking=True)

    done = torch.cuda.Event()
    done.record(s2)
    torch.cuda.synchronize()

    def plain(r):
        copy(r, r % 8)

    def record(r):
        copy(r, r % 8)
        torch.cuda.Event().record(s1)

    def wait_done(r):
        s1.wait_event(done)
        copy(r, r % 8)
        torch.cuda.Event().record(s1)

    def wait_fresh(r):
        ev = torch.cuda.Event()
        ev.record(s2)
        s1.wait_event(ev)
        copy(r, r % 8)
        torch.cuda.Event().record(s1)

    for rep in range(2):
        for name, body in (("plain", plain), ("event record after", record),
                           ("wait on a completed event", wait_done), ("wait on a fresh event", wait_fresh)):
            print(f"[prof_h2d] gaps, pass {rep}: 24 copies, {name}: {timed(24, body):.1f} us per copy", flush=True)
    for n_blobs in sorted({8, nl}):
        for order in ("in order", "stride 7"):
            step = 1 if order == "in order" else 7
            us = timed(64, lambda r: copy(r, (r * step) % n_blobs))
            print(f"[prof_h2d] working set {n_blobs} blobs ({n_blobs * BLOB / 1e9:.2f} GB), 64 copies {order}: "
                  f"{us:.1f} us per copy", flush=True)


if __name__ == "__main__":
    main()
