"""Driver for hardware-counter runs (rocprofv3 --pmc ...).

Runs a plain fp32 scale kernel over a buffer of known size (the calibration
for the byte counters), then one Llama-3.1-8B-shaped layer (NF4 base, LoRA
rank 16 on all seven projections, ``--tokens`` tokens as sequences of
``--seq``): forward, and the backward that recomputes it, ``--reps`` times.

    python3 bench/prof_layer.py [--reps 2] [--tokens 512] [--seq 512]
"""
import argparse
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from layer_streamed_frozen_amd import binding as B  # noqa: E402
from layer_streamed_frozen_amd import store as S  # noqa: E402
from layer_streamed_frozen_amd import synth  # noqa: E402


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=2)
    ap.add_argument("--tokens", type=int, default=512)
    ap.add_argument("--seq", type=int, default=512)
    args = ap.parse_args()
    if args.tokens % args.seq:
        raise SystemExit("--tokens must be a multiple of --seq")
    B.lib()
    torch.cuda.set_device(0)
    # calibration: reads 256 MiB and writes 256 MiB in one elementwise kernel
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    del src, dst

    shape = S.LLAMA8B
    W = S.layer_weights_fp32("prof.layer", shape)
    blob = S.build_layer_blob(shape, W)
    cfg = shape.cfg(args.tokens // args.seq, args.seq)
    lw = B.layer_weights_from_blob(cfg, B.FMT_NF4, blob.data_ptr())
    lora = S.LoraSet(shape, 1, prefix="prof.lora")
    H = shape.hidden
    x = torch.from_numpy(synth.bf16_exact(synth.normal("prof.x", (args.tokens, H)))[1].view(np.int16)) \
        .view(torch.bfloat16).cuda()
    dy = torch.from_numpy(synth.bf16_exact(synth.normal("prof.dy", (args.tokens, H)))[1].view(np.int16)) \
        .view(torch.bfloat16).cuda()
    ws = torch.empty(B.layer_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    ls = lora.struct(0)
    torch.cuda.synchronize()
    for r in range(args.reps):
        B.layer_fwd(cfg, lw, ls, x, y, ws)
        B.layer_bwd(cfg, lw, ls, x, dy, dx, ws)
        torch.cuda.synchronize()
        print(f"[prof_layer] rep {r} done", flush=True)


if __name__ == "__main__":
    main()
