"""The NVFP4 prep kernels form every quotient the format defines (block
amax / fl32(6G), and each element / D) as float(double(x) * r) with r a
double reciprocal of the float divisor instead of a float division: the
correctly rounded 1 / double(d) for the block scale, and for the elements
the hardware reciprocal refined by two Newton steps, which lies within one
double ulp of it.  This pins the identity that makes them equal,
float(x/d) == float(double(x) * r) for floats x, d and for r = 1/double(d)
and its two neighbouring doubles, on quotients placed as close as floats
allow to the midpoints between adjacent floats (the only places where two
roundings could part), with divisors across the normal and subnormal range,
next to plain random pairs.  numpy's float32 division is IEEE correctly
rounded, so it is the definition."""
import numpy as np


def _check(x, d):
    ok = np.isfinite(x) & (d != 0) & np.isfinite(d)
    x, d = x[ok], d[ok]
    r = 1.0 / d.astype(np.float64)
    with np.errstate(over="ignore"):   # quotients beyond the float range: inf on both sides
        want = np.divide(x, d, dtype=np.float32)
        for rr in (r, np.nextafter(r, np.inf), np.nextafter(r, -np.inf)):
            got = (x.astype(np.float64) * rr).astype(np.float32)
            bad = np.flatnonzero(want.view(np.uint32) != got.view(np.uint32))
            assert bad.size == 0, (x[bad[:5]], d[bad[:5]])
    return x.size


def test_quotients_next_to_float_midpoints():
    rng = np.random.default_rng(0)
    n = 1_000_000
    total = 0
    for lo, hi in ((-149, -126), (-126, 0), (0, 127)):   # subnormal, small and large divisors
        d = (rng.uniform(1, 2, n) * 2.0 ** rng.integers(lo, hi, n)).astype(np.float32)
        d = d[(d > 0) & np.isfinite(d)]
        q = (rng.uniform(1, 2, d.size) * 2.0 ** rng.integers(-12, 10, d.size)).astype(np.float32)
        mid = (q.astype(np.float64) + np.nextafter(q, np.float32(np.inf)).astype(np.float64)) / 2
        with np.errstate(over="ignore"):
            x = (mid * d.astype(np.float64)).astype(np.float32)
        for xx in (x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(-np.inf))):
            total += _check(np.where(rng.random(xx.size) < 0.5, xx, -xx), d)
    assert total > 8_000_000


def test_random_float_pairs():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=(2, 2_000_000), dtype=np.uint64).astype(np.uint32)
    assert _check(bits[0].view(np.float32), bits[1].view(np.float32)) > 1_000_000


def test_zero_divisor_matches_division():
    x = np.array([1.0, -2.5, 0.0, -0.0], np.float32)
    d = np.zeros(4, np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        want = np.divide(x, d, dtype=np.float32)
        got = (x.astype(np.float64) * (1.0 / d.astype(np.float64))).astype(np.float32)
    assert np.array_equal(np.isnan(want), np.isnan(got))
    assert np.array_equal(want[~np.isnan(want)], got[~np.isnan(got)])
