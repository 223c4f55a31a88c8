"""Host check of the quotient method the quantize kernels use.

The kernels take the fp32 quotient d / s (affine codes: (w - z) / s; nvfp4:
w / decoded scale) not by a division per element but as the fp64 product
d * r, r = 1/s correctly rounded in fp64, rounded to fp32. The argument that
this equals the IEEE fp32 quotient for every normal-range result is in the
kernel source; this test checks it numerically with numpy (IEEE fp32
division, IEEE fp64 arithmetic) on random operands across the exponent
range and on quotients placed on and around fp32 rounding midpoints.
Subnormal quotients are excluded: every caller maps them to code 0 or a
signed zero, whatever their last bit.
"""
import numpy as np

TINY = np.float32(np.finfo(np.float32).tiny)


def _method(d, s):
    r = np.float64(1.0) / s.astype(np.float64)
    return (d.astype(np.float64) * r).astype(np.float32)


def _check(d, s):
    with np.errstate(over="ignore", under="ignore", invalid="ignore", divide="ignore"):
        q = (d / s).astype(np.float32)
        m = _method(d, s)
    keep = np.isfinite(q) & (np.abs(q) >= TINY)
    bad = np.flatnonzero(keep & (q != m))
    assert bad.size == 0, (d[bad[:4]], s[bad[:4]], q[bad[:4]], m[bad[:4]])
    return int(keep.sum())


def test_random_operands_all_exponents():
    r = np.random.default_rng(2024)
    n = 2_000_000
    d = (r.standard_normal(n) * np.float32(2.0) ** r.integers(-100, 100, n)).astype(np.float32)
    s = (np.abs(r.standard_normal(n)) * np.float32(2.0) ** r.integers(-100, 100, n)).astype(np.float32)
    s[s == 0] = 1
    assert _check(d, s) > 0.8 * n      # the rest over- or underflow fp32


def test_random_significands_narrow_range():
    # quotients of O(1..255), as in affine codes: d in [0, n*s]
    r = np.random.default_rng(7)
    n = 2_000_000
    s = (r.random(n) * 0.01 + 1e-6).astype(np.float32)
    d = (r.random(n) * 255 * s).astype(np.float32)
    assert _check(d, s) > 0.9 * n


def test_quotients_near_midpoints():
    # d chosen so that d / s lands on, or within a few ulps of, a midpoint
    # between two fp32 values (the only place a second rounding could differ)
    r = np.random.default_rng(11)
    n = 500_000
    s = (1.0 + r.random(n)).astype(np.float32) * np.float32(2.0) ** r.integers(-40, 40, n).astype(np.float32)
    q = (1.0 + r.random(n)).astype(np.float32)
    mid = q.astype(np.float64) + np.spacing(q).astype(np.float64) / 2   # fp32 midpoint above q
    d0 = (mid * s.astype(np.float64)).astype(np.float32)
    total = 0
    for k in range(-3, 4):
        d = d0.copy()
        for _ in range(abs(k)):
            d = np.nextafter(d, np.float32(np.inf if k > 0 else -np.inf), dtype=np.float32)
        total += _check(d, s)
    assert total > 0.9 * 7 * n


def test_half_steps_of_small_scales():
    # the affine pins' groups: s = a * 2^-k, elements on half-steps and around
    for a, k in [(3, 0), (63, 4), (3, 6), (11, 2), (15, 9), (25, 3)]:
        s = np.float32(a * 2.0 ** -k)
        m = np.arange(255, dtype=np.float64)
        tie = ((m + 0.5) * np.float64(s)).astype(np.float32)
        ds = [tie]
        for step in (1, 2):
            ds.append(np.nextafter(ds[-1] if step == 1 else ds[-1], np.float32(np.inf), dtype=np.float32))
        lo = tie
        for _ in range(2):
            lo = np.nextafter(lo, np.float32(-np.inf), dtype=np.float32)
            ds.append(lo)
        d = np.concatenate(ds)
        _check(d, np.full(d.shape, s, np.float32))
