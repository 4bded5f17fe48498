"""Oracle: AdamW with 8-bit block-wise quantised moment states.

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

Source: the tutorial page (alphalab.site/soup-layer-streaming, section "step 2:
one YAML") configures the optimizer as ``paged_adamw_8bit``, and the benchmark
ledger it quotes (section on the published numbers) ran PagedAdamW8bit.  The
pages name the optimizer only.  Reading taken here: AdamW (the update of
``oracle/optim.py``) whose two moments are stored between steps in 8 bits with
block-wise dynamic quantisation, the published 8-bit optimizer method
(Dettmers et al., "8-bit Optimizers via Block-wise Quantization"): blocks of
2048 consecutive values, one fp32 absmax per block, each value stored as the
nearest entry of a fixed 8-bit code of [-1, 1] (first moment, signed) or
[0, 1] (second moment, unsigned) after division by the absmax.  Each step
dequantises, updates in fp32, and requantises with the new block absmax.
"Paged" (spilling state to host memory under pressure) does not change what is
computed and is not modelled.

The code (dynamic tree quantisation, as that method describes it): a value is
+-10^-E * f, where E is the number of zero bits that follow the sign bit, the
first one-bit after them is an indicator, and the remaining F bits give a
linear fraction f in (0.1, 1].  This oracle fixes the fraction as
f = 0.1 + 0.9 (j + 1) / 2^F for the F-bit index j, so f reaches 1 exactly:

* signed: 7 bits after the sign, E = 0..6, F = 6 - E: 127 positive values, their
  negatives and 0 (255 distinct values; the stored int8 code c in [-127, 127]
  is the value's position relative to 0 in the sorted table);
* unsigned: all 8 bits, E = 0..7, F = 7 - E: 255 positive values and 0 (the
  stored uint8 code is the position in the sorted table).

Values are formed in fp64 as (0.1 + 0.9 (j + 1) / 2^F) / 10^E and rounded to
fp32.  Quantisation takes the count of fp32 midpoints ((a + b) * 0.5 in fp32)
strictly below x / absmax (IEEE fp32 division): the nearest value, a tie going
to the smaller one; an all-zero block stores absmax 0 and the zero code.

The update runs in fp32 with every operation rounded (no fused multiply-add),
in this order, so that the GPU kernel can reproduce its codes exactly:

  g1 = g * f                       f: clip factor (1 when clipping is off)
  m0 = Ts[qm] * am,  v0 = Tu[qv] * av
  p1 = p - decay * p               decay = fp32(lr * wd)
  m1 = b1 * m0 + (1 - b1) * g1     (1 - b1) rounded in fp32
  v1 = b2 * v0 + (1 - b2) * (g1 * g1)
  p2 = p1 - step * (m1 / (sqrt(v1) * isb2 + eps))
       step = fp32(lr / (1 - b1^t)), isb2 = fp32(1 / sqrt(1 - b2^t)),
       b^t by repeated fp64 multiplication
  am', av' = block max of |m1|, v1; qm, qv = codes of m1 / am', v1 / av'.

Parity: pinned (closed-form table entries and counts, nearest-value
quantisation against brute force, the round-trip bound, the first step from
zero state against fp64 AdamW of ``oracle/optim.py``, a 30-step trajectory
staying within the code's resolution of fp64 AdamW).
"""
import numpy as np

BLOCK = 2048
F32 = np.float32


def dynamic_table(signed):
    """Sorted fp32 values of the signed (255 values) or unsigned (256) code."""
    bits = 7 if signed else 8
    pos = []
    for e in range(bits):
        nfrac = bits - 1 - e
        for j in range(2 ** nfrac):
            pos.append((0.1 + 0.9 * (j + 1) / 2.0 ** nfrac) / 10.0 ** e)
    pos = sorted(pos)
    vals = ([-x for x in reversed(pos)] + [0.0] + pos) if signed else ([0.0] + pos)
    return np.array(vals, dtype=np.float64).astype(F32)


def midpoints(table):
    """fp32 midpoints of consecutive table values."""
    return ((table[:-1] + table[1:]) * F32(0.5)).astype(F32)


def zero_index(signed):
    return 127 if signed else 0


def quantize(x, signed):
    """Block-wise codes and absmax of the fp32 vector x (blocks of BLOCK)."""
    x = np.asarray(x, F32)
    table = dynamic_table(signed)
    mids = midpoints(table)
    z = zero_index(signed)
    n = x.size
    nb = (n + BLOCK - 1) // BLOCK
    idx = np.empty(n, np.int64)
    absmax = np.zeros(nb, F32)
    for b in range(nb):
        blk = x[b * BLOCK:(b + 1) * BLOCK]
        a = F32(np.max(np.abs(blk))) if blk.size else F32(0)
        absmax[b] = a
        if a == 0:
            idx[b * BLOCK:(b + 1) * BLOCK] = z
        else:
            y = (blk / a).astype(F32)
            idx[b * BLOCK:(b + 1) * BLOCK] = np.searchsorted(mids, y, side="left")
    codes = (idx - z).astype(np.int8) if signed else idx.astype(np.uint8)
    return codes, absmax


def dequantize(codes, absmax, signed):
    """fp32 values table[code] * absmax[block]."""
    table = dynamic_table(signed)
    idx = codes.astype(np.int64) + zero_index(signed)
    blk = np.arange(codes.size) // BLOCK
    return (table[idx] * absmax[blk]).astype(F32)


def _pow_int(b, t):
    r = float(b)
    for _ in range(t - 1):
        r *= float(b)
    return r


def adamw8_step(p, g, qm, qv, am, av, t, lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                clip=1.0):
    """One update of the flat fp32 parameter vector p.  Hyper-parameters are
    taken as fp32 values; clip is the fp32 factor on the gradient.  Returns
    (p, qm, qv, am, av) after the step."""
    lr, beta1, beta2, eps = F32(lr), F32(beta1), F32(beta2), F32(eps)
    bc1 = 1.0 - _pow_int(beta1, t)
    bc2 = 1.0 - _pow_int(beta2, t)
    step = F32(float(lr) / bc1)
    isb2 = F32(1.0 / np.sqrt(bc2))
    decay = F32(float(lr) * float(weight_decay))
    omb1 = F32(F32(1) - beta1)
    omb2 = F32(F32(1) - beta2)
    p = np.asarray(p, F32)
    g1 = (np.asarray(g, F32) * F32(clip)).astype(F32)
    m0 = dequantize(qm, am, True)
    v0 = dequantize(qv, av, False)
    p1 = (p - (decay * p).astype(F32)).astype(F32)
    m1 = ((beta1 * m0).astype(F32) + (omb1 * g1).astype(F32)).astype(F32)
    v1 = ((beta2 * v0).astype(F32) + (omb2 * (g1 * g1).astype(F32)).astype(F32)).astype(F32)
    den = ((np.sqrt(v1).astype(F32) * isb2).astype(F32) + eps).astype(F32)
    p2 = (p1 - (step * (m1 / den).astype(F32)).astype(F32)).astype(F32)
    qm2, am2 = quantize(m1, True)
    qv2, av2 = quantize(v1, False)
    return p2, qm2, qv2, am2, av2
