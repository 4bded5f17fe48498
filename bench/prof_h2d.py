"""Host-to-device rate of one 8B-shaped NF4 layer blob (122,699,776 bytes)
copied on its own: from a pinned store of --layers such blobs into one of two
device buffers, one hipMemcpyAsync per copy, with and without a bf16 GEMM load
on another stream, and the same copy cut in two on two streams.

    python3 bench/prof_h2d.py [--layers 32] [--reps 64]

Prints, per variant, the median, minimum and maximum copy time (event-timed).
"""
import argparse
import statistics

import torch

BLOB = 122699776


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--reps", type=int, default=64)
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

    for busy in (False, True):
        for pieces in (1, 2):
            run(pieces, busy)  # warm
            ts = run(pieces, busy)
            med = statistics.median(ts)
            print(f"[prof_h2d] GEMM load on another stream: {busy}, streams: {pieces}: median {med:.0f} us "
                  f"({BLOB / med / 1e3:.2f} GB/s), min {min(ts):.0f}, max {max(ts):.0f}", flush=True)


if __name__ == "__main__":
    main()
