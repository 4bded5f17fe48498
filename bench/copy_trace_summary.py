"""Summarise the layer copies in a rocprofv3 memory-copy trace of a streamed
step (the `*_memory_copy_trace.csv` of `rocprofv3 --memory-copy-trace
--output-format csv`).

    python3 bench/copy_trace_summary.py TRACE.csv [--blob 122699776] [--pieces 2]

Layer copies are the host-to-device copies of 0.5 to 10 ms (the store build's
copies are shorter, the 1 GiB link-peak copies longer).  With --pieces N each
layer goes out as N consecutive pieces (the stack forks the second copy stream
from the first and joins it back before the next layer's copy), so every N
pieces in start order make one layer copy, timed from the first piece's start
to the last piece's end.  Prints the layer-copy durations and rates, how many
layers' pieces overlapped, the copy engines' idle gaps and busy fraction.
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
    if len(pieces) % n:
        raise SystemExit(f"{len(pieces)} layer-copy pieces is not a multiple of {n}")
    layers = [pieces[k:k + n] for k in range(0, len(pieces), n)]
    span = [max(p[1] for p in g) - min(p[0] for p in g) for g in layers]
    overlapped = sum(1 for g in layers if n > 1 and any(g[i + 1][0] < g[i][1] for i in range(n - 1)))
    starts = [min(p[0] for p in g) for g in layers]
    ends = [max(p[1] for p in g) for g in layers]
    gaps = [starts[k + 1] - ends[k] for k in range(len(layers) - 1)]
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
        print(f"idle between layer copies (gaps under 1 ms): {len(short)}, median {statistics.median(short) / 1e3:.1f} us, "
              f"{sum(short) / 1e6:.1f} ms in all")
    if long_:
        print(f"idle gaps over 1 ms: {len(long_)}, median {statistics.median(long_) / 1e6:.2f} ms")
    print(f"copy engines busy over the traced span: {sum(span) / (ends[-1] - starts[0]):.3f} "
          f"of {(ends[-1] - starts[0]) / 1e6:.1f} ms")
    print("layer copy durations (ms), in order: " + " ".join(f"{s / 1e6:.2f}" for s in span))


if __name__ == "__main__":
    main()
