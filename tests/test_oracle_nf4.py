"""Pins for the NF4 oracle: each test checks it against something other than
itself (the published table and its quantile construction, brute-force nearest
level, exact ties, closed-form bounds, hand-packed bytes, torch's bf16 cast)."""
import os

import numpy as np
import pytest
import torch

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nf4_codebook.txt")


def _golden():
    vals, bits = [], []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        _, v, b = line.split()
        vals.append(float(v))
        bits.append(int(b, 16))
    return np.array(vals, dtype=np.float32), np.array(bits, dtype=np.uint32)


def test_levels_match_published_table():
    vals, bits = _golden()
    assert vals.size == 16
    assert np.array_equal(nf4.nf4_levels().view(np.uint32), bits)
    assert np.array_equal(vals.view(np.uint32), bits)


def test_levels_structure():
    c = nf4.nf4_levels()
    assert c[0] == -1.0 and c[15] == 1.0
    assert c.view(np.uint32)[7] == 0            # exactly +0.0
    assert np.all(np.diff(c) > 0)
    assert np.count_nonzero(c < 0) == 7 and np.count_nonzero(c > 0) == 8


def test_levels_quantile_construction():
    # QLoRA's construction: standard-normal quantiles of an evenly spaced
    # probability grid from offset 0.9677083 down to 0.5 (9 points, last
    # dropped, for the 8 positive levels; 8 points for the 7 negative ones),
    # plus an exact zero, normalised by the maximum.
    from scipy.stats import norm
    off = 0.9677083
    p_pos = torch.linspace(off, 0.5, 9, dtype=torch.float32)[:-1].double().numpy()
    p_neg = torch.linspace(off, 0.5, 8, dtype=torch.float32)[:-1].double().numpy()
    v = np.sort(np.concatenate([norm.ppf(p_pos), [0.0], -norm.ppf(p_neg)]))
    v32 = v.astype(np.float32)
    v32 = v32 / v32.max()
    assert np.array_equal(v32, nf4.nf4_levels())
    assert np.max(np.abs(v / v.max() - nf4.nf4_levels())) < 1.1e-7


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        rng.standard_normal(1000).astype(np.float32) * 1e-30,
                        np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 0.0, -0.0],
                                 dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nf4.bf16_round(x), ref)
    # ties to even, by hand
    assert nf4.bf16_round(np.array([1 + 2 ** -8], np.float32))[0] == 0x3F80
    assert nf4.bf16_round(np.array([1 + 3 * 2 ** -8], np.float32))[0] == 0x3F82


def _blocks(nblocks, seed=0, std=0.02):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(nblocks * 64) * std).astype(np.float32)


def test_quantize_is_nearest_level():
    w = _blocks(4096)
    codes, absmax = nf4.nf4_codes(w)
    x = (w.reshape(-1, 64) / absmax[:, None]).astype(np.float32).reshape(-1)
    c = nf4.nf4_levels().astype(np.float64)
    dist = np.abs(x.astype(np.float64)[:, None] - c[None, :])
    nearest = np.argmin(dist, axis=1)
    # exact midpoints in real arithmetic; skip x within a few ulp of one
    mids = (c[:-1] + c[1:]) / 2
    near_tie = np.min(np.abs(x.astype(np.float64)[:, None] - mids[None, :]), axis=1) < 4e-7
    assert np.count_nonzero(near_tie) < 50
    assert np.array_equal(codes[~near_tie], nearest[~near_tie])


def test_exact_ties_go_to_lower_level():
    t = nf4.nf4_midpoints()
    for k in range(15):
        w = np.zeros(64, np.float32)
        w[0] = 1.0                          # absmax 1 -> x == w exactly
        w[1] = t[k]
        w[2] = np.nextafter(t[k], np.float32(2))
        w[3] = np.nextafter(t[k], np.float32(-2))
        codes, absmax = nf4.nf4_codes(w)
        assert absmax[0] == 1.0
        assert codes[1] == k, (k, codes[1])
        assert codes[2] == k + 1
        assert codes[3] == k


def test_extremes_and_zeros():
    w = _blocks(256, seed=3)
    codes, absmax = nf4.nf4_codes(w)
    blocks = w.reshape(-1, 64)
    arg = np.argmax(np.abs(blocks), axis=1)
    ext_codes = codes.reshape(-1, 64)[np.arange(blocks.shape[0]), arg]
    ext_vals = blocks[np.arange(blocks.shape[0]), arg]
    assert np.all(ext_codes == np.where(ext_vals > 0, 15, 0))
    deq = nf4.nf4_dequantize_f32(nf4.nf4_pack(codes), absmax).reshape(-1, 64)
    assert np.array_equal(deq[np.arange(blocks.shape[0]), arg], ext_vals)  # exactly +-absmax
    # a zero element maps to level 0.0 and dequantises to exactly 0
    w2 = w.copy()
    w2[5] = 0.0
    c2, a2 = nf4.nf4_codes(w2)
    assert c2[5] == 7
    assert nf4.nf4_dequantize_f32(nf4.nf4_pack(c2), a2)[5] == 0.0


def test_all_zero_block():
    w = np.zeros(128, np.float32)
    w[64:] = _blocks(1, seed=4)
    codes, absmax = nf4.nf4_codes(w)
    assert absmax[0] == 0.0 and np.all(codes[:64] == 7)
    bits = nf4.nf4_dequantize_bf16(nf4.nf4_pack(codes), absmax)
    assert np.all(bits[:64] == 0)


def test_requantize_is_idempotent():
    w = _blocks(2048, seed=5)
    p, a = nf4.nf4_quantize(w)
    deq = nf4.nf4_dequantize_f32(p, a)
    p2, a2 = nf4.nf4_quantize(deq)
    assert np.array_equal(a2, a)
    assert np.array_equal(p2, p)


def test_round_trip_bound():
    w = _blocks(4096, seed=6)
    p, a = nf4.nf4_quantize(w)
    half_gap = np.max(np.diff(nf4.nf4_levels().astype(np.float64))) / 2
    assert abs(half_gap - 0.15190360) < 1e-7
    scale = np.repeat(a, 64).astype(np.float64)
    err = np.abs(w - nf4.nf4_dequantize_f32(p, a).astype(np.float64))
    assert np.all(err <= half_gap * scale * (1 + 2 ** -22) + 1e-30)
    # bf16 keeps 8 significant bits: one RNE rounding adds at most 2^-8 of |c * absmax|
    errb = np.abs(w - nf4.bf16_to_f32(nf4.nf4_dequantize_bf16(p, a)).astype(np.float64))
    assert np.all(errb <= (half_gap + 2 ** -8) * scale * (1 + 2 ** -20))


def test_pack_nibble_order():
    codes = np.array([1, 2, 3, 4, 15, 0], np.uint8)
    assert list(nf4.nf4_pack(codes)) == [0x12, 0x34, 0xF0]
    rng = np.random.default_rng(8)
    c = rng.integers(0, 16, 4096).astype(np.uint8)
    assert np.array_equal(nf4.nf4_unpack(nf4.nf4_pack(c)), c)


def test_blocks_follow_row_major_flattening():
    w = _blocks(8, seed=9).reshape(4, 128)      # two blocks per row
    _, absmax = nf4.nf4_codes(w)
    ref = np.max(np.abs(w.reshape(4, 2, 64)), axis=2).reshape(-1)
    assert np.array_equal(absmax, ref)


def test_rejects_ragged_size():
    with pytest.raises(ValueError):
        nf4.nf4_codes(np.zeros(100, np.float32))


# ------------------------------------------------------ double quantisation

def test_dq_keeps_single_level_codes():
    w = _blocks(1000, seed=20)
    p1, a1 = nf4.nf4_quantize(w)
    p2, aq, s2, a2 = nf4.nf4dq_quantize(w)
    assert np.array_equal(p1, p2) and np.array_equal(a1, a2)
    assert aq.size == 1000 and s2.shape == (4, 2)   # 1000 blocks -> 4 groups, the last ragged


def test_dq_code_is_nearest_of_256_levels():
    a = np.abs(np.random.default_rng(21).standard_normal(256 * 3).astype(np.float32)) * 0.05
    codes, s2 = nf4.dq_encode_absmax(a)
    for gi in range(3):
        scale, off = s2[gi].astype(np.float64)
        levels = (np.arange(256, dtype=np.float32) * np.float32(s2[gi, 0])).astype(np.float32) + np.float32(s2[gi, 1])
        grp = a[gi * 256:(gi + 1) * 256].astype(np.float64)
        d = np.abs(grp[:, None] - levels[None, :].astype(np.float64))
        best = np.argmin(d, axis=1)
        gap = np.sort(d, axis=1)
        clear = (gap[:, 1] - gap[:, 0]) > 1e-6 * scale   # skip near-ties
        assert np.array_equal(codes[gi * 256:(gi + 1) * 256][clear], best[clear])


def test_dq_group_minimum_exact_and_error_bound():
    a = np.abs(np.random.default_rng(22).standard_normal(256 * 2 + 17).astype(np.float32)) * 0.03
    codes, s2 = nf4.dq_encode_absmax(a)
    ad = nf4.dq_decode_absmax(codes, s2)
    for gi in range(3):
        grp = slice(gi * 256, min(a.size, (gi + 1) * 256))
        i = np.argmin(a[grp])
        assert ad[grp][i] == a[grp][i]                       # the offset itself
        assert codes[grp].max() == 255
        scale = np.float64(s2[gi, 0])
        assert np.all(np.abs(ad[grp].astype(np.float64) - a[grp]) <= scale / 2 * (1 + 1e-5) + 1e-9)


def test_dq_constant_group():
    a = np.full(300, 0.0421, np.float32)
    codes, s2 = nf4.dq_encode_absmax(a)
    assert np.all(codes == 0) and np.all(s2[:, 0] == 0)
    assert np.array_equal(nf4.dq_decode_absmax(codes, s2), a)


def test_dq_dequant_close_to_single_level():
    w = _blocks(512, seed=23)
    p, aq, s2, am = nf4.nf4dq_quantize(w)
    d1 = nf4.nf4_dequantize_f32(p, am).astype(np.float64)
    d2 = nf4.bf16_to_f32(nf4.nf4dq_dequantize_bf16(p, aq, s2)).astype(np.float64)
    assert np.linalg.norm(d2 - d1) / np.linalg.norm(d1) < 1e-2
