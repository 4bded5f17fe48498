"""Shared helpers of the test suite (comparison metrics, oracle inputs)."""
import numpy as np
import torch

from layer_streamed_frozen_amd import synth
from oracle import nf4 as onf4

TOL = 2e-2  # relative Frobenius error bound for bf16 results against the fp64 oracle
ROW_TOL = 5e-2  # bound on every row's relative error (rows: the last axis of the result)
ROW_FLOOR = 0.5  # a row's error is measured against at least this fraction of the RMS row norm


def rel_fro(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


def worst_row(got, ref):
    """Largest per-row relative error (rows = last axis; a 1-D result is one
    value per row).  Each row is measured against max(its own norm,
    ROW_FLOOR x the RMS row norm), so rows that are legitimately tiny are not
    judged by their own noise, while a handful of bad rows in a large result
    cannot hide under the overall Frobenius figure."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    g = g.reshape(-1, g.shape[-1]) if g.ndim >= 2 else g.reshape(-1, 1)
    r = r.reshape(g.shape)
    rn = np.linalg.norm(r, axis=1)
    floor = ROW_FLOOR * np.sqrt(np.mean(rn * rn))
    den = np.maximum(rn, max(floor, 1e-300))
    err = np.linalg.norm(g - r, axis=1) / den
    i = int(np.argmax(err))
    rms = np.sqrt(np.mean(rn * rn))
    return float(err[i]), i, float(rn[i] / rms) if rms > 0 else 0.0


def report(name, got, ref):
    """Print the relative Frobenius error, the largest absolute error and the
    worst row; assert the worst row is within ROW_TOL; return the Frobenius
    error (callers compare it with TOL)."""
    e, m = rel_fro(got, ref), max_abs(got, ref)
    w, i, rel_norm = worst_row(got, ref)
    print(f"  {name:>10s}: rel_fro={e:.3e} max_abs={m:.3e} worst_row={w:.3e} (row {i}, norm {rel_norm:.2f} x RMS)",
          flush=True)
    assert w < ROW_TOL, f"{name}: row {i} relative error {w:.3e} >= {ROW_TOL}"
    return e


def report_sum(name, got, ref, part):
    """Like report, for a result that is the sum of two parts computed with
    bf16 rounding, ref = part + (ref - part), which may cancel (the DPO
    adapter gradients: chosen minus rejected sequences).  Each part held to
    TOL bounds the error of the sum by TOL (|part| + |ref - part|) (triangle
    inequality), so that is the scale, overall and per row (with the row floor
    of worst_row).  Returns the error over that scale."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    a = np.asarray(part, dtype=np.float64)
    b = r - a
    scale = np.linalg.norm(a) + np.linalg.norm(b)
    e = float(np.linalg.norm(g - r) / max(scale, 1e-300))
    g2, r2 = g.reshape(-1, g.shape[-1]), r.reshape(-1, r.shape[-1])
    a2, b2 = a.reshape(g2.shape), b.reshape(g2.shape)
    rs = np.linalg.norm(a2, axis=1) + np.linalg.norm(b2, axis=1)
    rms = np.sqrt(np.mean(rs * rs))
    err = np.linalg.norm(g2 - r2, axis=1) / np.maximum(rs, max(ROW_FLOOR * rms, 1e-300))
    i = int(np.argmax(err))
    print(f"  {name:>10s}: err/(|part|+|rest|)={e:.3e} rel_fro={rel_fro(g, r):.3e} "
          f"cancellation={scale / max(np.linalg.norm(r), 1e-300):.2f} worst_row={err[i]:.3e} (row {i})", flush=True)
    assert err[i] < ROW_TOL, f"{name}: row {i} error {err[i]:.3e} >= {ROW_TOL} of |part| + |rest|"
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
