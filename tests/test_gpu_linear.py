"""GPU parity of one NF4 linear layer with a LoRA adapter (forward and
backward) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from layer_streamed_frozen_amd import binding as B
from layer_streamed_frozen_amd import synth
from oracle import model as M
from tests._util import TOL, bf16_input, bf16_tensor_to_np, oracle_dense, report

pytestmark = pytest.mark.gpu


def _run(prefix, n_out, n_in, T, r, alpha, b_zero=False, adapter=True):
    print(f"[linear] {prefix} out={n_out} in={n_in} T={T} r={r}", flush=True)
    s = alpha / r
    W = synth.normal(f"{prefix}.W", (n_out, n_in), 0.02)
    lim = 1.0 / np.sqrt(n_in)
    A = synth.uniform(f"{prefix}.A", (r, n_in), -lim, lim)
    Bm = np.zeros((n_out, r), np.float32) if b_zero else synth.normal(f"{prefix}.B", (n_out, r), 0.01)
    X, xg = bf16_input(f"{prefix}.X", (T, n_in))
    dY, dyg = bf16_input(f"{prefix}.dY", (T, n_out))

    wd = torch.from_numpy(W.reshape(-1)).cuda()
    packed, absmax = B.nf4_quantize(wd)
    w = B.weight(packed, absmax)
    Ag = torch.from_numpy(A).cuda() if adapter else None
    Bg = torch.from_numpy(Bm).cuda() if adapter else None
    ws = torch.empty(B.linear_workspace_bytes(T, n_out, n_in, r), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, n_out), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((T, n_in), dtype=torch.bfloat16, device="cuda")
    dA = torch.zeros((r, n_in), dtype=torch.float32, device="cuda")
    dB = torch.zeros((n_out, r), dtype=torch.float32, device="cuda")
    B.linear_fwd(w, B.FMT_NF4, n_out, n_in, Ag, Bg, r, s, xg, y, ws)
    B.linear_bwd(w, B.FMT_NF4, n_out, n_in, Ag, Bg, r, s, xg, dyg, dx, dA if adapter else None,
                 dB if adapter else None, ws)
    torch.cuda.synchronize()

    Wd = oracle_dense(W)
    X64, dY64 = X.astype(np.float64), dY.astype(np.float64)
    A64, B64 = (A.astype(np.float64), Bm.astype(np.float64)) if adapter else (None, None)
    yr, u = M.lora_linear_fwd(X64, Wd, A64, B64, s)
    dxr, dAr, dBr = M.lora_linear_bwd(dY64, X64, Wd, A64, B64, s, u)
    out = dict(y=(bf16_tensor_to_np(y), yr), dx=(bf16_tensor_to_np(dx), dxr))
    if adapter:
        out["dA"] = (dA.double().cpu().numpy(), dAr)
        out["dB"] = (dB.double().cpu().numpy(), dBr)
    return out


def test_single_linear_config():
    # 256x256 weight, rank 8, alpha 16, 64 tokens
    res = _run("cfg1", 256, 256, 64, 8, 16.0)
    for k, (g, r) in res.items():
        assert report(k, g, r) < TOL, k


def test_linear_several_tiles_ragged_tokens():
    res = _run("lin2", 384, 640, 200, 16, 16.0)
    for k, (g, r) in res.items():
        assert report(k, g, r) < TOL, k


def test_linear_long_contraction_split_k():
    res = _run("lin3", 256, 4096, 70, 4, 8.0)
    for k, (g, r) in res.items():
        assert report(k, g, r) < TOL, k


def test_wide_forward_kernel_matches_oracle_and_general_kernel():
    # 16384 outputs, 2048 inputs: the forward GEMM runs on the ping-pong
    # kernel (one ragged 512-row tile), and so does the input gradient (a
    # contraction over 16384, 8 splits); the general kernels give the same
    # bits.
    n0 = B.gemm_wide_launch_count()
    res = _run("linwide", 16384, 2048, 300, 16, 16.0)
    assert B.gemm_wide_launch_count() == n0 + 2
    for k, (g, r) in res.items():
        assert report(k, g, r) < TOL, k
    B.gemm_set_wide(False)
    try:
        res2 = _run("linwide", 16384, 2048, 300, 16, 16.0)
    finally:
        B.gemm_set_wide(True)
    assert B.gemm_wide_launch_count() == n0 + 2
    for k in res:
        assert np.array_equal(res[k][0], res2[k][0]), k


@pytest.mark.parametrize("n_out,n_in,T", [(4096, 14336, 512), (6144, 8192, 300), (2048, 8192, 257)])
def test_wide_split_k_matches_oracle_and_general_kernel(n_out, n_in, T):
    # Long contractions over few 512 x 128 tiles (32, 48, 16): the forward
    # GEMM runs split-K on the ping-pong kernel (8, 5, 8 splits), fp32 partial
    # sums then the ordered reduction.  The second case has a shorter last
    # split (48 of 52 k tiles), the others a ragged row tile; the LoRA steps
    # ride on the last split.  The input gradient (8192 or 14336 outputs) runs
    # split-K on the input-gradient ping-pong kernel (2, 4, 4 splits).  The
    # general kernels with the same splits give the same bits.
    n0 = B.gemm_wide_launch_count()
    res = _run(f"linsk{n_out}", n_out, n_in, T, 16, 16.0)
    assert B.gemm_wide_launch_count() == n0 + 2
    for k, (g, r) in res.items():
        assert report(k, g, r) < TOL, k
    B.gemm_set_wide(False)
    try:
        res2 = _run(f"linsk{n_out}", n_out, n_in, T, 16, 16.0)
    finally:
        B.gemm_set_wide(True)
    assert B.gemm_wide_launch_count() == n0 + 2
    for k in res:
        assert np.array_equal(res[k][0], res2[k][0]), k


def test_wide_kernel_chosen_by_tile_count():
    # 6144 outputs (the q|k|v width) over 2048 tokens: 8 x 24 = 192 tiles of
    # 256 x 256, enough for the wide kernel; it matches the oracle and gives the
    # general kernel's bits.
    n0 = B.gemm_wide_launch_count()
    res = _run("linwq", 6144, 2048, 2048, 16, 16.0)
    assert B.gemm_wide_launch_count() == n0 + 1
    for k, (g, r) in res.items():
        assert report(k, g, r) < TOL, k
    B.gemm_set_wide(False)
    try:
        res2 = _run("linwq", 6144, 2048, 2048, 16, 16.0)
    finally:
        B.gemm_set_wide(True)
    for k in res:
        assert np.array_equal(res[k][0], res2[k][0]), k
    # 512 tokens of the same width: 48 tiles, and a contraction too short for
    # split-K on the wide kernel: the general kernel
    n1 = B.gemm_wide_launch_count()
    _run("linwq5", 6144, 2048, 512, 16, 16.0)
    assert B.gemm_wide_launch_count() == n1


def test_b_zero_reproduces_base_output_bitwise():
    a = _run("lin4", 256, 512, 96, 16, 16.0, b_zero=True)
    b = _run("lin4", 256, 512, 96, 16, 16.0, adapter=False)
    assert np.array_equal(a["y"][0], b["y"][0])
    assert np.all(a["dA"][0] == 0.0)
