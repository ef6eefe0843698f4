"""Pin the oracle's binary32 sigmoid (router scores are sigmoids: "Reflection
Releases Beam ...", section "Where Beam Saves and Where the Memory Bill Comes
In") against a 60-digit decimal evaluation rounded to binary32.

The oracle evaluates in binary64 (Cody-Waite reduction + degree-13 Taylor)
and rounds once, so it must equal the correctly rounded value everywhere
except where the exact sigmoid lies within a few binary64 ulps of a binary32
rounding boundary.  A dropped ln2 tail, a wrong sign, a short polynomial or a
wrong reduction constant each break equality on many of these inputs.
"""
import numpy as np
import pytest

import oracle
from oracle.bruteforce import sigmoid32_exact

NEAR = 1e-15  # relative distance to a binary32 midpoint treated as a near-tie


def _inputs():
    rng = np.random.default_rng(1234)
    parts = [
        rng.uniform(-8, 8, 12000),
        rng.uniform(-30, 30, 6000),
        rng.uniform(-110, 50, 3000),
        rng.standard_normal(6000) * 1.0,          # router logits have std ~1
        np.array([0.0, -0.0, 1e-30, -1e-30, 1e-7, -1e-7, 0.5, -0.5, 1.0, -1.0,
                  16.5, 17.0, 17.5, 39.99, 40.0, 41.0, -87.0, -87.5, -88.7,
                  -100.0, -103.9, -103.97, -103.98, -104.0, -104.5, -150.0,
                  1e6, -1e6]),
    ]
    v = np.concatenate(parts).astype(np.float32)
    # all binary32 neighbours of a few points
    for c in (0.0, 1.0, -1.0, 2.0, -17.0):
        a = np.float32(c)
        for _ in range(20):
            a = np.nextafter(a, np.float32(np.inf))
            v = np.append(v, a)
    return v


def test_sigmoid32_is_correctly_rounded():
    v = _inputs()
    got = oracle.sigmoid32(v)
    near = 0
    bad = []
    for x, g in zip(v, got):
        want, margin = sigmoid32_exact(float(x))
        if margin < NEAR:
            near += 1
            continue
        if g.view(np.uint32) != want.view(np.uint32):
            bad.append((float(x), float(g), float(want)))
    assert not bad, f"{len(bad)} mismatches, first {bad[:5]}"
    assert near <= 3, near


def test_sigmoid32_special_values():
    v = np.array([0.0, -200.0, 200.0, -104.0, 40.0], np.float32)
    s = oracle.sigmoid32(v)
    assert s[0] == np.float32(0.5)
    assert s[1] == 0.0 and not np.signbit(s[1])
    assert s[2] == 1.0
    assert s[3] == 0.0
    assert s[4] == 1.0


def test_sigmoid32_symmetry_within_rounding():
    # s(x) + s(-x) = 1 exactly in the reals; after one rounding each, the sum
    # is within one ulp of 1 for moderate |x|.
    rng = np.random.default_rng(7)
    v = rng.uniform(-10, 10, 2000).astype(np.float32)
    a = oracle.sigmoid32(v).astype(np.float64)
    b = oracle.sigmoid32(-v).astype(np.float64)
    assert np.max(np.abs(a + b - 1.0)) <= 2.0 ** -24 * 1.0001


def test_sigmoid_binary64_error_bound():
    # Before rounding to binary32, the binary64 value is within a few binary64
    # ulps of the exact sigmoid (a short polynomial or a coarse ln2 split
    # would leave errors far above 1e-15).
    from fractions import Fraction
    from oracle.bruteforce import exact_sigmoid
    rng = np.random.default_rng(99)
    v = np.concatenate([rng.uniform(-103, 39, 3000), rng.standard_normal(3000) * 3,
                        np.linspace(-0.36, 0.36, 101)]).astype(np.float32)
    q = oracle.sigmoid_f64(v)
    worst = 0.0
    for x, a in zip(v, q):
        e = exact_sigmoid(float(x))
        worst = max(worst, float(abs(Fraction(float(a)) - e) / e))
    assert worst < 1e-15, worst
