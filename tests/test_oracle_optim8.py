"""Pins for the 8-bit-state AdamW oracle."""
import numpy as np

from oracle import optim as O
from oracle import optim8 as Q


def test_signed_table_closed_forms():
    t = Q.dynamic_table(True)
    assert t.dtype == np.float32 and t.size == 255
    assert np.all(np.diff(t.astype(np.float64)) > 0)
    assert t[127] == 0.0 and t[254] == 1.0 and t[0] == -1.0
    np.testing.assert_array_equal(t, -t[::-1])
    # largest values: the 64 fractions of the first decade, 1/64 of 0.9 apart
    assert t[253] == np.float32(0.1 + 0.9 * 63 / 64)
    assert t[191] == np.float32(0.1 + 0.9 / 64)
    # smallest positive: the last decade has a single value, 1e-6
    assert t[128] == np.float32(1e-6)
    pos = t[128:].astype(np.float64)
    for e, count in enumerate([64, 32, 16, 8, 4, 2, 1]):
        lo, hi = 10.0 ** -(e + 1), 10.0 ** -e
        assert np.sum((pos > lo * (1 + 1e-7)) & (pos <= hi * (1 + 1e-7))) == count, e


def test_unsigned_table_closed_forms():
    t = Q.dynamic_table(False)
    assert t.size == 256 and t[0] == 0.0 and t[255] == 1.0
    assert np.all(np.diff(t.astype(np.float64)) > 0)
    assert t[1] == np.float32(1e-7)
    assert t[254] == np.float32(0.1 + 0.9 * 127 / 128)
    assert np.sum(t >= np.float32(0.1 + 0.9 / 128)) == 128


def _brute_nearest(y, table):
    """Nearest table index by exhaustive fp64 distances, and whether the two
    nearest are too close to call (y within fp32 rounding of their midpoint,
    where the documented rule - fp32 midpoints, tie to the smaller value -
    may pick either)."""
    d = np.abs(y.astype(np.float64)[:, None] - table.astype(np.float64)[None, :])
    order = np.argsort(d, axis=1, kind="stable")
    first, second = order[:, 0], order[:, 1]
    d1 = d[np.arange(y.size), first]
    d2 = d[np.arange(y.size), second]
    close = (d2 - d1) <= 2 ** -23 * np.maximum(np.abs(y.astype(np.float64)), 1e-30)
    return first, second, close


def test_quantize_is_nearest_value_by_brute_force():
    rng = np.random.default_rng(80)
    for signed in (True, False):
        table = Q.dynamic_table(signed)
        z = Q.zero_index(signed)
        # mix of magnitudes across every decade, exact table values and midpoints
        y = rng.uniform(-1 if signed else 0, 1, 3000) * (10.0 ** -rng.integers(0, 8, 3000))
        mids = Q.midpoints(table).astype(np.float64)
        y = np.concatenate([y, table.astype(np.float64), mids]).astype(np.float32)
        if not signed:
            y = np.abs(y)
        y[0] = 1.0  # the block maximum
        codes, absmax = Q.quantize(y, signed)
        assert absmax[0] == np.max(np.abs(y[:Q.BLOCK]))
        for b in range(absmax.size):
            blk = y[b * Q.BLOCK:(b + 1) * Q.BLOCK]
            yy = (blk / absmax[b]).astype(np.float32)
            first, second, close = _brute_nearest(yy, table)
            got = codes[b * Q.BLOCK:(b + 1) * Q.BLOCK].astype(np.int64) + z
            np.testing.assert_array_equal(got[~close], first[~close])
            assert np.all((got[close] == first[close]) | (got[close] == second[close]))
            # only the inserted midpoints (and a stray random value or two) are ties
            assert np.sum(close) <= (mids.size if b == absmax.size - 1 else 0) + 3


def test_round_trip_bound_and_exact_extremes():
    rng = np.random.default_rng(81)
    x = (rng.standard_normal(5000) * 3e-3).astype(np.float32)
    for signed in (True, False):
        xs = x if signed else np.abs(x)
        codes, absmax = Q.quantize(xs, signed)
        back = Q.dequantize(codes, absmax, signed)
        table = Q.dynamic_table(signed).astype(np.float64)
        gap = np.max(np.diff(table)) / 2  # largest half-spacing (near 1)
        blk = np.arange(xs.size) // Q.BLOCK
        err = np.abs(back.astype(np.float64) - xs)
        assert np.all(err <= absmax[blk].astype(np.float64) * (gap + 1e-7))
        # each block's largest magnitude comes back exactly
        for b in range(absmax.size):
            i = b * Q.BLOCK + np.argmax(np.abs(xs[b * Q.BLOCK:(b + 1) * Q.BLOCK]))
            assert back[i] == xs[i]
    zero_codes, zero_max = Q.quantize(np.zeros(3000, np.float32), True)
    assert np.all(zero_codes == 0) and np.all(zero_max == 0)


def test_first_step_from_zero_state_matches_fp64_adamw():
    rng = np.random.default_rng(82)
    n = 2 * Q.BLOCK + 333
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    qm, am = Q.quantize(np.zeros(n, np.float32), True)
    qv, av = Q.quantize(np.zeros(n, np.float32), False)
    kw = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    p8, qm8, qv8, am8, av8 = Q.adamw8_step(p, g, qm, qv, am, av, 1, **kw)
    # fp32 hyper-parameters, as the fp32 path sees them
    kw64 = {k: float(np.float32(v)) for k, v in kw.items()}
    pr, mr, vr, _ = O.adamw_step([p.astype(np.float64)], [g.astype(np.float64)], [np.zeros(n)], [np.zeros(n)], 1,
                                 **kw64)
    # fp32 storage of p: at most two roundings of p's own size apart
    np.testing.assert_allclose(p8, pr[0], rtol=2.5e-7, atol=1e-10)
    # the stored states are the new moments up to the code's resolution
    m8 = Q.dequantize(qm8, am8, True).astype(np.float64)
    v8 = Q.dequantize(qv8, av8, False).astype(np.float64)
    blk = np.arange(n) // Q.BLOCK
    assert np.all(np.abs(m8 - mr[0]) <= am8[blk] * 0.0071 + 1e-12)
    assert np.all(np.abs(v8 - vr[0]) <= av8[blk] * 0.0036 + 1e-18)


def test_trajectory_tracks_fp64_adamw():
    # A quadratic bowl: g = p - target.  The 8-bit states change the path only
    # by the code's resolution, so 30 steps stay close to the exact optimizer.
    rng = np.random.default_rng(83)
    n = Q.BLOCK + 500
    target = (rng.standard_normal(n) * 0.05).astype(np.float32)
    p8 = np.zeros(n, np.float32)
    qm, am = Q.quantize(np.zeros(n, np.float32), True)
    qv, av = Q.quantize(np.zeros(n, np.float32), False)
    pr, mr, vr = [np.zeros(n)], [np.zeros(n)], [np.zeros(n)]
    lr = 1e-3
    for t in range(1, 31):
        g8 = (p8 - target).astype(np.float32)
        p8, qm, qv, am, av = Q.adamw8_step(p8, g8, qm, qv, am, av, t, lr=lr)
        gr = [pr[0] - target.astype(np.float64)]
        pr, mr, vr, _ = O.adamw_step(pr, gr, mr, vr, t, lr=float(np.float32(lr)))
    # The code's resolution is about 1.4% of the block absmax in the top decade
    # and coarser relative to smaller values, so individual paths drift by a
    # few percent (median 5% here); the distance left to the target agrees.
    moved = np.abs(pr[0])
    diff = np.abs(p8.astype(np.float64) - pr[0])
    assert np.max(moved) > 0.02
    assert np.max(diff) < 0.25 * np.max(moved)
    assert np.median(diff) < 0.1 * np.median(moved)
    d8 = np.linalg.norm(p8.astype(np.float64) - target)
    dr = np.linalg.norm(pr[0] - target)
    assert abs(d8 - dr) < 0.05 * dr and dr < 0.7 * np.linalg.norm(target)


def test_zero_gradient_and_zero_state_only_decays():
    p = np.linspace(-1, 1, 3001).astype(np.float32)
    qm, am = Q.quantize(np.zeros(p.size, np.float32), True)
    qv, av = Q.quantize(np.zeros(p.size, np.float32), False)
    p2, qm2, qv2, am2, av2 = Q.adamw8_step(p, np.zeros_like(p), qm, qv, am, av, 3, lr=1e-2, weight_decay=0.5)
    decay = np.float32(float(np.float32(1e-2)) * 0.5)
    np.testing.assert_array_equal(p2, (p - decay * p).astype(np.float32))
    assert np.all(qm2 == 0) and np.all(qv2 == 0) and np.all(am2 == 0) and np.all(av2 == 0)
