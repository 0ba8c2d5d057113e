"""Pins of the oracle's sigmoid against mathematics it does not share.

The oracle claims s = RN32(1 / (1 + e^-x)). These tests check that claim with
mpmath at 50 digits (nearest binary32 by exact distance comparison), with
closed forms, and with monotonicity.
"""
import mpmath
import numpy as np
import pytest

import oracle as O

mpmath.mp.dps = 50


def _nearest_ok(x: np.float32, f: np.float32) -> bool:
    """True iff f is the binary32 nearest to sigma(x), by exact comparison."""
    xs = mpmath.mpf(float(x))
    sig = 1 / (1 + mpmath.exp(-xs))
    up = np.nextafter(f, np.float32(np.inf))
    dn = np.nextafter(f, np.float32(-np.inf))
    d0 = abs(sig - mpmath.mpf(float(f)))
    d_up = abs(sig - mpmath.mpf(float(up)))
    d_dn = abs(sig - mpmath.mpf(float(dn))) if f > 0 else mpmath.mpf("inf")
    return d0 < d_up and d0 < d_dn


def test_sigmoid_zero_is_half():
    assert O.sigmoid_rn32(np.array([0.0, -0.0], np.float32)).tolist() == [0.5, 0.5]


def test_sigmoid_saturates_to_one_and_zero():
    # 1 - sigma(x) = 1 / (1 + e^x) < 2^-25 for x >= 17.33: rounds to 1.0.
    big = np.array([17.5, 20.0, 88.0, 1e4, 3.0e38], np.float32)
    assert np.all(O.sigmoid_rn32(big) == np.float32(1.0))
    # sigma(x) < e^x < 2^-150 for x <= -104: rounds to +0.
    tiny = np.array([-104.5, -200.0, -1e4, -3.0e38], np.float32)
    out = O.sigmoid_rn32(tiny)
    assert np.all(out == 0.0) and not np.any(np.signbit(out))


def test_sigmoid_matches_mpmath_random():
    rng = np.random.default_rng(1234)
    xs = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (4.0 * rng.standard_normal(2000)).astype(np.float32),
        rng.uniform(-110.0, 20.0, 2000).astype(np.float32),   # includes subnormal results
        rng.uniform(-1e-3, 1e-3, 500).astype(np.float32),
    ])
    out = O.sigmoid_rn32(xs)
    bad = [(float(x), float(f)) for x, f in zip(xs, out) if not _nearest_ok(x, f)]
    assert not bad, bad[:5]


def test_sigmoid_matches_mpmath_near_rounding_boundaries():
    """Hardest inputs of a 2^22-point sweep: binary64 sigmoid closest to a
    binary32 midpoint. The expected rounding comes from mpmath only."""
    u = np.arange(0, 2 ** 22, dtype=np.uint32) * np.uint32(1021) + np.uint32(0x3E000000)
    x = u.view(np.float32)
    x = np.concatenate([x, -x])
    x = x[np.isfinite(x) & (np.abs(x) < 60)]
    d = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    f = d.astype(np.float32)
    ulp = np.nextafter(f, np.float32(np.inf)).astype(np.float64) - f.astype(np.float64)
    # distance of d from the nearest midpoint, in units of the binary32 ulp
    frac = np.abs(np.abs(d - f.astype(np.float64)) / ulp - 0.5)
    hard = np.argsort(frac)[:300]
    out = O.sigmoid_rn32(x[hard])
    bad = [float(v) for v, f0 in zip(x[hard], out) if not _nearest_ok(v, f0)]
    assert not bad, bad[:5]


def test_sigmoid_subnormal_range_matches_mpmath():
    xs = np.linspace(-103.9, -86.0, 400).astype(np.float32)
    out = O.sigmoid_rn32(xs)
    assert np.any(out < np.finfo(np.float32).tiny)  # subnormals really occur
    bad = [float(x) for x, f in zip(xs, out) if not _nearest_ok(x, f)]
    assert not bad, bad[:5]


def test_sigmoid_monotone_nondecreasing():
    u = np.arange(0x3F000000, 0x42000000, 997, dtype=np.uint32)  # 0.5 .. 32
    pos = u.view(np.float32)
    x = np.concatenate([-pos[::-1], np.array([0.0], np.float32), pos])
    s = O.sigmoid_rn32(x)
    assert np.all(np.diff(s.astype(np.float64)) >= 0.0)


def test_sigmoid_fallbacks_are_rare():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(1 << 20).astype(np.float32)
    n = O.sigmoid_rn32_fallback_count(x)
    assert n < 200  # about 2^-15.5 of inputs expected


@pytest.mark.parametrize("mutant", ["plain_fp32", "truncate"])
def test_planted_sigmoid_mistakes_are_caught(mutant):
    """A plausible wrong sigmoid (fp32 evaluation, or truncation instead of
    round-to-nearest) fails the mpmath pin."""
    rng = np.random.default_rng(99)
    xs = rng.standard_normal(3000).astype(np.float32)
    if mutant == "plain_fp32":
        with np.errstate(over="ignore"):
            out = (np.float32(1.0) / (np.float32(1.0) + np.exp(-xs))).astype(np.float32)
    else:
        d = 1.0 / (1.0 + np.exp(-xs.astype(np.float64)))
        out = (d.astype(np.float32))
        over = out.astype(np.float64) > d
        out[over] = np.nextafter(out[over], np.float32(0))
    bad = sum(1 for x, f in zip(xs, out) if not _nearest_ok(x, f))
    assert bad > 0
