"""Host-to-device rate of one 8B-shaped NF4 layer blob (122,699,776 bytes)
copied on its own: from a pinned store of --layers such blobs into one of two
device buffers, one hipMemcpyAsync per copy, with and without a bf16 GEMM load
on another stream, and the same copy cut in two on two streams.

    python3 bench/prof_h2d.py [--layers 32] [--reps 64] [--sustain SECONDS [--idle]] [--probe-gaps]

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
order and in a stride-7 order.
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
    args = ap.parse_args()
    nl = args.layers
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
