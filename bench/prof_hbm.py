"""Driver for the HBM-bound kernels' counter and trace runs (rocprofv3).

Runs a plain fp32 scale kernel over a buffer of known size (the calibration
for the byte counters), then, ``--reps`` times each:

* nf4_quantize and nf4_dequantize of one 28672 x 4096 weight (the gate|up
  projection of an 8B-shaped layer: 117 M weights);
* layer_fwd and the recomputing layer_bwd of one Llama-3.1-8B-shaped NF4 layer
  (LoRA rank 16 on all seven projections) at ``--tokens`` tokens (default
  16384 = 32 sequences of 512), large enough that RMSNorm, RoPE and the
  split-K reductions are no longer launch-bound.

    python3 bench/prof_hbm.py [--reps 3] [--tokens 16384]
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
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--tokens", type=int, default=16384)
    args = ap.parse_args()
    if args.tokens % 512:
        raise SystemExit("--tokens must be a multiple of 512")
    B.lib()
    torch.cuda.set_device(0)
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    print("[prof_hbm] calibration done", flush=True)

    n = 28672 * 4096
    w = torch.from_numpy(synth.normal("prof.hbm.w", (n,), 0.02)).cuda()
    packed = torch.empty(n // 2, dtype=torch.uint8, device="cuda")
    absmax = torch.empty(n // 64, dtype=torch.float32, device="cuda")
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    for r in range(args.reps):
        B.nf4_quantize(w, packed, absmax)
        B.nf4_dequantize(packed, absmax, n, out)
    torch.cuda.synchronize()
    del w, packed, absmax, out
    print("[prof_hbm] quantize / dequantize done", flush=True)

    shape = S.LLAMA8B
    W = S.layer_weights_fp32("prof.layer", shape)
    blob = S.build_layer_blob(shape, W)
    cfg = shape.cfg(args.tokens // 512, 512)
    lw = B.layer_weights_from_blob(cfg, B.FMT_NF4, blob.data_ptr())
    lora = S.LoraSet(shape, 1, prefix="prof.lora")
    H = shape.hidden
    x = torch.from_numpy(synth.bf16_exact(synth.normal("prof.hbm.x", (args.tokens, H)))[1].view(np.int16)) \
        .view(torch.bfloat16).cuda()
    dy = torch.from_numpy(synth.bf16_exact(synth.normal("prof.hbm.dy", (args.tokens, H)))[1].view(np.int16)) \
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
        print(f"[prof_hbm] layer rep {r} done", flush=True)


if __name__ == "__main__":
    main()
