"""Summarise the layer copies in a rocprofv3 memory-copy trace of a streamed
step (the `*_memory_copy_trace.csv` of `rocprofv3 --memory-copy-trace
--output-format csv`).

    python3 bench/copy_trace_summary.py TRACE.csv [--blob 122699776] [--pieces 2]

Layer copies are the host-to-device copies of 0.5 to 10 ms (the store build's
copies are shorter, the 1 GiB link-peak copies longer).  With --pieces N each
layer goes out as N pieces, one on each of N copy streams, each stream carrying
its pieces in layer order; the k-th piece of every stream make layer copy k,
timed from the first piece's start to the last piece's end.  Prints the
layer-copy durations and rates, how many layers' pieces overlapped, and the
idle gaps and busy fraction of the copy engines together (time in which no
piece of any layer copy is in flight, which also holds when one stream's next
layer starts before the other stream's piece of this one ends).
"""
import argparse
import csv
import statistics


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("trace")
    ap.add_argument("--blob", type=int, default=122699776)
    ap.add_argument("--pieces", type=int, default=2)
    a = ap.parse_args()
    rows = [r for r in csv.DictReader(open(a.trace)) if r["Direction"] == "MEMORY_COPY_HOST_TO_DEVICE"]
    c = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Stream_Id"]) for r in rows)
    pieces = [x for x in c if 500_000 < x[1] - x[0] < 10_000_000]
    n = a.pieces
    by_stream = {}
    for p in pieces:
        by_stream.setdefault(p[2], []).append(p)
    if len(by_stream) != n or len({len(v) for v in by_stream.values()}) != 1:
        raise SystemExit(f"expected {n} streams with one piece per layer each, found "
                         f"{ {k: len(v) for k, v in by_stream.items()} }")
    # every copy stream carries one piece of every layer, in layer order
    layers = sorted(sorted(g) for g in zip(*(sorted(v) for v in by_stream.values())))
    span = [max(p[1] for p in g) - min(p[0] for p in g) for g in layers]
    overlapped = sum(1 for g in layers if n > 1 and any(g[i + 1][0] < g[i][1] for i in range(n - 1)))
    busy_iv = []  # union of the pieces' intervals
    for p in sorted(pieces):
        if busy_iv and p[0] <= busy_iv[-1][1]:
            busy_iv[-1][1] = max(busy_iv[-1][1], p[1])
        else:
            busy_iv.append([p[0], p[1]])
    gaps = [busy_iv[k + 1][0] - busy_iv[k][1] for k in range(len(busy_iv) - 1)]
    t0, t1 = busy_iv[0][0], busy_iv[-1][1]
    short = [g for g in gaps if g < 1_000_000]
    long_ = [g for g in gaps if g >= 1_000_000]
    gbps = lambda ns: a.blob / (ns * 1e-9) / 1e9  # noqa: E731
    med = statistics.median(span)
    print(f"layer copies {len(layers)} ({len(pieces)} pieces on streams {sorted({p[2] for p in pieces})}); "
          f"pieces overlapping in {overlapped}, one after another in {len(layers) - overlapped}")
    print(f"layer copy median / mean / min / max: {med / 1e3:.1f} / {statistics.mean(span) / 1e3:.1f} / "
          f"{min(span) / 1e3:.1f} / {max(span) / 1e3:.1f} us")
    print(f"rate of the median copy {gbps(med):.2f} GB/s, best {gbps(min(span)):.2f}, over all copies "
          f"{a.blob * len(span) / (sum(span) * 1e-9) / 1e9:.2f}")
    bins = [0] * 5
    for s in span:
        ms = s / 1e6
        bins[0 if ms < 2.2 else 1 if ms < 2.5 else 2 if ms < 3.2 else 3 if ms < 3.5 else 4] += 1
    print("layer copies under 2.2 ms / 2.2 - 2.5 / 2.5 - 3.2 / 3.2 - 3.5 / over 3.5 ms: "
          + " / ".join(str(b) for b in bins))
    if short:
        print(f"idle gaps under 1 ms: {len(short)}, median {statistics.median(short) / 1e3:.1f} us, "
              f"{sum(short) / 1e6:.1f} ms in all")
    if long_:
        print(f"idle gaps over 1 ms: {len(long_)}, median {statistics.median(long_) / 1e6:.2f} ms")
    busy = sum(e - b for b, e in busy_iv)
    print(f"copy engines busy over the traced span: {busy / (t1 - t0):.3f} of {(t1 - t0) / 1e6:.1f} ms")
    total = a.blob * len(layers)
    print(f"layer bytes over the busy time {total / (busy * 1e-9) / 1e9:.2f} GB/s, over the traced span "
          f"{total / ((t1 - t0) * 1e-9) / 1e9:.2f} GB/s")
    print("layer copy durations (ms), in order: " + " ".join(f"{s / 1e6:.2f}" for s in span))


if __name__ == "__main__":
    main()
