"""Oracle: blockwise NF4 (4-bit NormalFloat) quantise, pack and dequantise.

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

Source of the method: the tutorial "alphalab.site/soup-layer-streaming",
section "four-stage data path", item 1 (NF4): the decoder's quantisable Linear
weights are stored offline as QLoRA NF4; norms and the untied head stay in
higher precision, and compute runs in higher precision.  The pages name QLoRA's
NF4 but print neither its levels nor its block layout; the readings taken here
(all fixed in fp32, because every code is an integer decided by an fp32
comparison) are:

1. Levels: the 16 published NF4 values of QLoRA (Dettmers et al. 2023,
   Appendix E), ascending, as fp32.  They are stored verbatim in
   ``tests/golden/nf4_codebook.txt`` and checked against the quantile
   construction there.
2. Blocks of 64 consecutive elements of the row-major flattened weight, one
   fp32 absmax (max |w|) per block.
3. x = w / absmax with IEEE correctly-rounded fp32 division; code = number of
   fp32 midpoints t_k = fp32((c_k + c_{k+1}) / 2) with x > t_k.  The strict
   comparison sends an exact tie to the lower level.  An all-zero block keeps
   absmax 0 and every code 7 (the level 0.0).
4. Packing: byte j holds element 2j in its high nibble and 2j+1 in its low one.
5. Dequant: w' = bf16_rne(fp32(c[code] * absmax)).

Parity: pinned (codebook golden + construction, brute-force nearest level,
exact ties, extremes, idempotence, round-trip bound, hand-packed nibbles).
"""
import numpy as np

# The published NF4 levels (QLoRA, Appendix E), as fp32.
NF4_LEVELS = np.array([
    -1.0, -0.6961928009986877, -0.5250730514526367, -0.39491748809814453,
    -0.28444138169288635, -0.18477343022823334, -0.09105003625154495, 0.0,
    0.07958029955625534, 0.16093020141124725, 0.24611230194568634,
    0.33791524171829224, 0.44070982933044434, 0.5626170039176941,
    0.7229568362236023, 1.0], dtype=np.float32)

BLOCKSIZE = 64
ZERO_CODE = 7


def nf4_levels():
    """The 16 NF4 levels, fp32, ascending."""
    return NF4_LEVELS.copy()


def nf4_midpoints():
    """The 15 decision thresholds t_k = fp32((c_k + c_{k+1}) * 0.5)."""
    c = NF4_LEVELS
    return ((c[:-1] + c[1:]) * np.float32(0.5)).astype(np.float32)


def bf16_round(x):
    """Round fp32 values to the nearest bfloat16 (ties to even).

    Returns the uint16 bit patterns.  Finite inputs only (the method never
    produces NaN or Inf here).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return (r & np.uint64(0xFFFF)).astype(np.uint16)


def bf16_to_f32(bits):
    """Widen bfloat16 bit patterns (uint16) to fp32 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def nf4_codes(w, blocksize=BLOCKSIZE):
    """Quantise a weight to NF4 codes.

    w: any-shaped fp32 array whose size is a multiple of ``blocksize``;
    blocks run along the row-major flattening.
    Returns (codes uint8 [n], absmax fp32 [n / blocksize]).
    """
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    if w.size % blocksize:
        raise ValueError("element count must be a multiple of the block size")
    blocks = w.reshape(-1, blocksize)
    absmax = np.max(np.abs(blocks), axis=1).astype(np.float32)
    t = nf4_midpoints()
    codes = np.full(blocks.shape, ZERO_CODE, dtype=np.uint8)
    nz = absmax > 0
    if np.any(nz):
        x = (blocks[nz] / absmax[nz, None]).astype(np.float32)  # IEEE fp32 divide
        c = np.zeros(x.shape, dtype=np.uint8)
        for k in range(15):
            c += (x > t[k]).astype(np.uint8)
        codes[nz] = c
    return codes.reshape(-1), absmax


def nf4_pack(codes):
    """Pack codes two per byte: element 2j -> high nibble, 2j+1 -> low nibble."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    if codes.size % 2:
        raise ValueError("need an even number of codes")
    return ((codes[0::2] << 4) | codes[1::2]).astype(np.uint8)


def nf4_unpack(packed):
    """Inverse of ``nf4_pack``."""
    p = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p >> 4
    out[1::2] = p & 0x0F
    return out


def nf4_quantize(w, blocksize=BLOCKSIZE):
    """Quantise and pack.  Returns (packed uint8 [n/2], absmax fp32 [n/bs])."""
    codes, absmax = nf4_codes(w, blocksize)
    return nf4_pack(codes), absmax


def nf4_dequantize_f32(packed, absmax, blocksize=BLOCKSIZE):
    """fp32 product c[code] * absmax for every element (flat array)."""
    codes = nf4_unpack(packed)
    scale = np.repeat(np.asarray(absmax, dtype=np.float32), blocksize)
    if scale.size != codes.size:
        raise ValueError("absmax count does not match the packed size")
    return (NF4_LEVELS[codes] * scale).astype(np.float32)


def nf4_dequantize_bf16(packed, absmax, blocksize=BLOCKSIZE):
    """Dequantised weight as bfloat16 bit patterns (uint16, flat)."""
    return bf16_round(nf4_dequantize_f32(packed, absmax, blocksize))


def nf4_dequantize(packed, absmax, shape, blocksize=BLOCKSIZE):
    """Dequantised weight as the fp32 values of its bf16 rounding, reshaped."""
    return bf16_to_f32(nf4_dequantize_bf16(packed, absmax, blocksize)).reshape(shape)


# ------------------------------------------------------ double quantisation
#
# The pages' store and buffer sizes (3.60 GB over 32 layers, 113 MB per layer;
# review "repodaily.xyz/zh/projects/2026-08-17/soup/", architecture section)
# fit NF4 codes plus an 8-bit absmax, QLoRA's "double quantisation", but the
# pages do not give the second-level code.  Reading taken here (plain affine
# 8-bit, no codebook): the fp32 absmax values are grouped 256 at a time (in
# block order); per group offset = min, scale = fp32((max - min) / 255);
# code = clamp(rint(fp32(fp32(a - offset) / scale)), 0, 255) with
# round-half-to-even (code 0 when scale is 0).  The stored absmax is
# a' = fp32(fp32(code * scale) + offset).  NF4 codes are still chosen against
# the exact absmax; only the scale that dequantisation multiplies by is a'.
#
# Parity: pinned (NF4 codes equal the single-level ones; brute-force nearest
# of the 256 levels; group minimum reconstructs exactly; error bound scale/2).

DQ_GROUP = 256


def dq_encode_absmax(absmax):
    """8-bit codes of the absmax values and the per-group (scale, offset).

    Returns (codes uint8 [nb], scale2 fp32 [ngroups, 2]) with columns
    (scale, offset)."""
    a = np.ascontiguousarray(absmax, dtype=np.float32).reshape(-1)
    ng = (a.size + DQ_GROUP - 1) // DQ_GROUP
    codes = np.zeros(a.size, dtype=np.uint8)
    s2 = np.zeros((ng, 2), dtype=np.float32)
    for gi in range(ng):
        grp = a[gi * DQ_GROUP:(gi + 1) * DQ_GROUP]
        lo, hi = np.float32(grp.min()), np.float32(grp.max())
        scale = np.float32((hi - lo) / np.float32(255.0))
        if scale > 0:
            q = np.rint(((grp - lo).astype(np.float32) / scale).astype(np.float32))
            codes[gi * DQ_GROUP:gi * DQ_GROUP + grp.size] = np.clip(q, 0, 255).astype(np.uint8)
        s2[gi] = (scale, lo)
    return codes, s2


def dq_decode_absmax(codes, scale2):
    """a' = fp32(fp32(code * scale) + offset) for every block."""
    c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    g = np.arange(c.size) // DQ_GROUP
    scale = scale2[g, 0].astype(np.float32)
    off = scale2[g, 1].astype(np.float32)
    return ((c.astype(np.float32) * scale).astype(np.float32) + off).astype(np.float32)


def nf4dq_quantize(w, blocksize=BLOCKSIZE):
    """NF4 with a double-quantised absmax.

    Returns (packed uint8 [n/2], absmax codes uint8 [n/bs], scale2 fp32
    [ceil(n/bs/256), 2], exact absmax fp32 [n/bs])."""
    codes, absmax = nf4_codes(w, blocksize)
    aq, s2 = dq_encode_absmax(absmax)
    return nf4_pack(codes), aq, s2, absmax


def nf4dq_dequantize_bf16(packed, absq, scale2, blocksize=BLOCKSIZE):
    """bf16 bits of c[code] * a' (flat)."""
    return nf4_dequantize_bf16(packed, dq_decode_absmax(absq, scale2), blocksize)


def nf4dq_dequantize(packed, absq, scale2, shape, blocksize=BLOCKSIZE):
    return bf16_to_f32(nf4dq_dequantize_bf16(packed, absq, scale2, blocksize)).reshape(shape)
