"""The allocation-free single-linear forward (linear_fwd_noalloc) against
linear_fwd with a caller workspace, through the C ABI: the same bits on two
calls in a row, the second smaller than the first (the library's scratch
keeps the first call's contents), and the size limit refused up front."""
import ctypes

import numpy as np
import pytest
import torch

from layer_streamed_frozen_amd import binding as B
from layer_streamed_frozen_amd import synth
from tests._util import bf16_input

pytestmark = pytest.mark.gpu


def _case(prefix, n_out, n_in, T, r, adapter=True):
    W = synth.normal(f"{prefix}.W", (n_out, n_in), 0.02)
    packed, absmax = B.nf4_quantize(torch.from_numpy(W.reshape(-1)).cuda())
    w = B.weight(packed, absmax)
    lim = 1.0 / np.sqrt(n_in)
    A = torch.from_numpy(synth.uniform(f"{prefix}.A", (r, n_in), -lim, lim)).cuda() if adapter else None
    Bm = torch.from_numpy(synth.normal(f"{prefix}.B", (n_out, r), 0.01)).cuda() if adapter else None
    _, x = bf16_input(f"{prefix}.X", (T, n_in))
    return w, A, Bm, x


def _both(w, A, Bm, x, n_out, n_in, r, scale=2.0):
    T = x.shape[0]
    ws = torch.empty(B.linear_workspace_bytes(T, n_out, n_in, r), dtype=torch.uint8, device="cuda")
    y_ws = torch.full((T, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    y_na = torch.full((T, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.linear_fwd(w, B.FMT_NF4, n_out, n_in, A, Bm, r, scale, x, y_ws, ws)
    B.linear_fwd_noalloc(w, B.FMT_NF4, n_out, n_in, A, Bm, r, scale, x, y_na)
    torch.cuda.synchronize()
    return y_ws, y_na


def test_noalloc_matches_workspace_call_twice_then_smaller():
    print("[noalloc] 512 x 1024 x 1024 r16, then 64 x 256 x 256 r8, then 200 x 384 x 640 no adapter", flush=True)
    big = (1024, 1024, 16)
    y1, z1 = _both(*_case("na.big", big[0], big[1], 512, big[2]), *big)
    assert torch.isfinite(y1.float()).all()
    assert torch.equal(y1, z1)
    small = (256, 256, 8)
    y2, z2 = _both(*_case("na.small", small[0], small[1], 64, small[2]), *small)
    assert torch.isfinite(y2.float()).all()
    assert torch.equal(y2, z2)
    third = (384, 640, 16)
    y3, z3 = _both(*_case("na.plain", third[0], third[1], 200, third[2], adapter=False), *third)
    assert torch.equal(y3, z3)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    cap = B.linear_noalloc_max_bytes()
    assert cap == 32 << 20
    # 8 split-K partials of T x N fp32 exceed 32 MiB at T = 512, N = 4096
    assert B.linear_workspace_bytes(512, 4096, 4096, 16) > cap
    w, A, Bm, x = _case("na.huge", 4096, 256, 512, 16)
    y = torch.empty((512, 4096), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.LsfError) as e:
        B.linear_fwd_noalloc(w, B.FMT_NF4, 4096, 256, A, Bm, 16, 1.0, x, y)
    assert e.value.status == B.LSF_ERR_WORKSPACE
    assert "32" in str(e.value) or "bytes" in str(e.value)
