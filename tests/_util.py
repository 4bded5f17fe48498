"""Shared helpers of the test suite (comparison metrics, oracle inputs)."""
import numpy as np
import torch

from layer_streamed_frozen_amd import synth
from oracle import nf4 as onf4

TOL = 2e-2  # relative Frobenius error bound for bf16 results against the fp64 oracle


def rel_fro(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


def report(name, got, ref):
    e, m = rel_fro(got, ref), max_abs(got, ref)
    print(f"  {name:>10s}: rel_fro={e:.3e} max_abs={m:.3e}", flush=True)
    return e


def bf16_tensor_to_np(t):
    """bf16 torch tensor -> fp64 numpy values."""
    return t.float().cpu().numpy().astype(np.float64)


def bf16_input(name, shape, std=1.0):
    """Seeded bf16-exact input: (fp32 numpy values, bf16 device tensor)."""
    vals, bits = synth.bf16_exact(synth.normal(name, shape, std))
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return vals, t


def oracle_dense(W):
    """The oracle's own NF4 round trip of a fp32 weight: dense fp64 [out, in]."""
    p, a = onf4.nf4_quantize(W)
    return onf4.nf4_dequantize(p, a, W.shape).astype(np.float64)


def oracle_dense_dq(W):
    """The oracle's double-quantised NF4 round trip: dense fp64 [out, in]."""
    p, aq, s2, _ = onf4.nf4dq_quantize(W)
    return onf4.nf4dq_dequantize(p, aq, s2, W.shape).astype(np.float64)


def oracle_dense_bf16(W):
    """An unquantised bf16 weight (its values are already bf16-exact)."""
    return np.asarray(W, dtype=np.float64)
