"""The memory-copy trace summariser on small synthetic traces whose figures
follow by hand: pieces paired per stream in layer order (also when one
stream runs ahead of the other), busy time as the union of pieces in flight."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TOOL = os.path.join(ROOT, "bench", "copy_trace_summary.py")
HEADER = '"Kind","Direction","Stream_Id","Source_Agent_Id","Destination_Agent_Id","Correlation_Id",' \
         '"Start_Timestamp","End_Timestamp"\n'


def write_trace(path, copies):
    with open(path, "w") as f:
        f.write(HEADER)
        for k, (stream, t0, t1) in enumerate(copies):
            f.write(f'"MEMORY_COPY","MEMORY_COPY_HOST_TO_DEVICE",{stream},"Agent 0","Agent 1",{k},{t0},{t1}\n')


def run(path, pieces):
    out = subprocess.run([sys.executable, TOOL, path, "--pieces", str(pieces), "--blob", "1000000"],
                         capture_output=True, text=True, check=True).stdout
    return out.splitlines()


def line(lines, prefix):
    hit = [ln for ln in lines if ln.startswith(prefix)]
    assert len(hit) == 1, (prefix, lines)
    return hit[0]


MS = 1_000_000  # ns


def test_two_streams_one_running_ahead(tmp_path):
    # stream 1: layer 0 at [0, 2] ms, layer 1 at [3, 5]; stream 3: layer 0 at [0, 1], layer 1 at [1, 3]
    # (stream 3 starts layer 1 before stream 1's layer 0 ends); a short store-build copy and a long
    # link-peak copy are ignored
    p = str(tmp_path / "t.csv")
    write_trace(p, [(1, 0, 2 * MS), (3, 0, 1 * MS), (3, 1 * MS, 3 * MS), (1, 3 * MS, 5 * MS),
                    (1, -50 * MS, -50 * MS + 1000), (1, -40 * MS, -20 * MS)])
    r = run(p, 2)
    # layer 0's halves [0, 2] and [0, 1] overlap; layer 1's [1, 3] and [3, 5] follow one another
    assert line(r, "layer copies 2") == ("layer copies 2 (4 pieces on streams ['1', '3']); pieces overlapping in 1, "
                                       "one after another in 1")
    # layer 0 spans [0, 2], layer 1 spans [1, 5]
    assert line(r, "layer copy median").endswith("3000.0 / 3000.0 / 2000.0 / 4000.0 us")
    # union of pieces in flight: [0, 5] ms without a gap
    assert line(r, "copy engines busy") == "copy engines busy over the traced span: 1.000 of 5.0 ms"
    # 2 layers x 1e6 bytes over 5 ms
    assert line(r, "layer bytes") == "layer bytes over the busy time 0.40 GB/s, over the traced span 0.40 GB/s"


def test_one_stream_gaps(tmp_path):
    p = str(tmp_path / "t.csv")
    # three copies of 1 ms with 0.1 ms and 2 ms gaps between them
    write_trace(p, [(2, 0, MS), (2, MS + MS // 10, 2 * MS + MS // 10), (2, 4 * MS + MS // 10, 5 * MS + MS // 10)])
    r = run(p, 1)
    assert line(r, "idle gaps under") == "idle gaps under 1 ms: 1, median 100.0 us, 0.1 ms in all"
    assert line(r, "idle gaps over") == "idle gaps over 1 ms: 1, median 2.00 ms"
    assert line(r, "copy engines busy") == "copy engines busy over the traced span: 0.588 of 5.1 ms"


def test_stream_count_must_match(tmp_path):
    p = str(tmp_path / "t.csv")
    write_trace(p, [(1, 0, MS), (3, 0, MS)])
    res = subprocess.run([sys.executable, TOOL, p, "--pieces", "1"], capture_output=True, text=True)
    assert res.returncode != 0 and "expected 1 streams" in (res.stderr + res.stdout)
