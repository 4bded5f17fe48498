"""GPU parity of NF4 quantise / dequantise: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from layer_streamed_frozen_amd import binding as B
from layer_streamed_frozen_amd import synth
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu


def _gpu_roundtrip(w):
    wd = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32).reshape(-1)).cuda()
    packed, absmax = B.nf4_quantize(wd)
    deq = B.nf4_dequantize(packed, absmax, wd.numel())
    torch.cuda.synchronize()
    return (packed.cpu().numpy(), absmax.cpu().numpy(),
            deq.view(torch.int16).cpu().numpy().view(np.uint16))


def _check(w, label):
    print(f"[nf4] {label} n={w.size}", flush=True)
    p, a, d = _gpu_roundtrip(w)
    rp, ra = onf4.nf4_quantize(w)
    assert np.array_equal(a.view(np.uint32), ra.view(np.uint32)), f"{label}: absmax differs"
    bad = np.nonzero(p != rp)[0]
    assert bad.size == 0, f"{label}: {bad.size} packed bytes differ, first at {bad[:5]}"
    rd = onf4.nf4_dequantize_bf16(rp, ra)
    assert np.array_equal(d, rd), f"{label}: dequantised bf16 differs"


def test_single_linear_weight():
    _check(synth.normal("cfg1.W", (256, 256), 0.02), "256x256")


def test_8b_o_projection_full():
    _check(synth.normal("nf4.o8b", (4096, 4096), 0.02), "4096x4096")


def test_8b_qkv_rows_concatenated():
    w = synth.normal("nf4.qkv8b", (6144, 4096), 0.02)
    _check(w, "6144x4096")


def test_smallest_and_ragged_counts():
    _check(synth.normal("nf4.tiny", (64,), 1.0), "one block")
    _check(synth.normal("nf4.odd", (64 * 37,), 1.0), "37 blocks")
    with pytest.raises(B.LsfError) as e:
        B.nf4_quantize(torch.zeros(100, device="cuda"))
    assert e.value.status == B.LSF_ERR_SHAPE


def test_adversarial_blocks():
    t = onf4.nf4_midpoints()
    blocks = []
    for k in range(15):  # exact ties and their neighbours, absmax exactly 1
        b = np.zeros(64, np.float32)
        b[0] = 1.0
        b[1] = t[k]
        b[2] = np.nextafter(t[k], np.float32(2))
        b[3] = np.nextafter(t[k], np.float32(-2))
        b[4] = -t[k]
        blocks.append(b)
    blocks.append(np.zeros(64, np.float32))                       # all zero
    b = np.zeros(64, np.float32); b[7] = -3.5; blocks.append(b)   # one negative extreme
    b = np.full(64, -0.0, np.float32); b[63] = 2.0; blocks.append(b)
    rng = np.random.default_rng(0)
    blocks.append((rng.standard_normal(64) * 1e30).astype(np.float32))
    blocks.append((rng.standard_normal(64) * 1e-20).astype(np.float32))
    blocks.append(np.linspace(-1, 1, 64, dtype=np.float32))
    blocks.append(np.full(64, 0.37, np.float32))                  # constant block
    # ties for a non-unit absmax: w = t_k * a computed in fp32 lands near the midpoint
    a = np.float32(0.0123)
    b = np.zeros(64, np.float32); b[0] = a; b[1:16] = t * a; blocks.append(b)
    _check(np.concatenate(blocks), "adversarial")


def test_denormal_blocks():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal(64 * 4) * 1e-39).astype(np.float32)
    _check(w, "denormal")


def _check_dq(w, label):
    print(f"[nf4dq] {label} n={w.size}", flush=True)
    wd = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32).reshape(-1)).cuda()
    packed, absmax, absq, s2 = B.nf4dq_quantize(wd)
    deq = B.nf4dq_dequantize(packed, absq, s2, wd.numel())
    torch.cuda.synchronize()
    rp, raq, rs2, ra = onf4.nf4dq_quantize(w)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), ra.view(np.uint32)), label
    assert np.array_equal(packed.cpu().numpy(), rp), label
    assert np.array_equal(s2.cpu().numpy().view(np.uint32), rs2.view(np.uint32)), f"{label}: scale/offset differ"
    bad = np.nonzero(absq.cpu().numpy() != raq)[0]
    assert bad.size == 0, f"{label}: {bad.size} absmax codes differ, first {bad[:5]}"
    rd = onf4.nf4dq_dequantize_bf16(rp, raq, rs2)
    assert np.array_equal(deq.view(torch.int16).cpu().numpy().view(np.uint16), rd), label


def test_dq_8b_o_projection_full():
    _check_dq(synth.normal("nf4.o8b", (4096, 4096), 0.02), "4096x4096")


def test_dq_ragged_groups_and_constant_group():
    _check_dq(synth.normal("nf4dq.odd", (64 * 300,), 0.5), "300 blocks")
    w = np.tile(np.linspace(-1, 1, 64, dtype=np.float32), 256)   # 256 identical blocks: scale 0
    _check_dq(w, "constant group")
