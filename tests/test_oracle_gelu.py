"""Pins for the oracle's INT8 -> INT8 GELU (CPU only).

Method: non-linear operators also read and write INT8 tensors with per-block
scales, because they are memory-bound (Jetfire summary, "Problem" and
"Approach").  Reading pinned here: x = fl(s*q), g = x*Phi(x) evaluated in
binary64 and rounded once to binary32, then per-block requantization.

References: mpmath at 50 significant digits (an arbitrary-precision erfc
that shares nothing with the C library), closed forms of GELU, and the exact
quantization rule.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle
from exact import frac, to_f32
from test_oracle_quant import exact_quantize_block

mpmath.mp.dps = 50


def gelu_exact_f32(x: float) -> Fraction:
    """Correctly rounded binary32 of x*Phi(x), Phi(x) = erfc(-x/sqrt(2))/2."""
    xm = mpmath.mpf(float(x))
    g = xm * mpmath.erfc(-xm / mpmath.sqrt(2)) / 2
    if g == 0:
        return Fraction(0)
    sign, man, exp, _ = g._mpf_
    return to_f32((-1) ** sign * Fraction(int(man)) * Fraction(2) ** int(exp))


def sample_points():
    g = np.random.default_rng(5)
    pts = [0.0, -0.0, 1e-30, -1e-30, 0.5, -0.5, -0.7518, 1.0, -1.0, 3.0, -3.0, 5.5, -5.5,
           8.0, -8.0, 10.0, -10.0, 12.0, -12.0, 40.0, -40.0, 127.0, -127.0, 3.0e4, -3.0e4]
    pts += list(g.standard_normal(300).astype(np.float32) * 3)
    s = np.float32(0.0231)
    pts += [float(s * np.float32(c)) for c in range(-127, 128)]
    return [float(np.float32(p)) for p in pts]


def test_gelu_value_is_correctly_rounded_binary32():
    for x in sample_points():
        assert frac(oracle.gelu_value(x)) == gelu_exact_f32(x), x


def test_closed_forms():
    # g(0) = 0; g(x) - g(-x) = x; g(x) = x for large x; g(x) -> 0 from below
    assert oracle.gelu_value(0.0) == 0.0
    for x in [0.25, 0.75, 1.5, 2.0, 4.0]:
        d = oracle.gelu_value(x) - oracle.gelu_value(-x)
        assert abs(d - x) <= 2 * np.spacing(np.float32(x)), x
    for x in [6.0, 9.5, 100.0, 1e6]:
        assert oracle.gelu_value(x) == np.float32(x)
    for x in [-6.0, -9.5, -30.0]:
        v = oracle.gelu_value(x)
        assert v <= 0.0 and abs(v) < 1e-8
    # the global minimum of x*Phi(x) is -0.16997... near x = -0.7518
    xs = np.linspace(-1.5, 0.0, 3001, dtype=np.float32)
    vals = np.array([oracle.gelu_value(float(x)) for x in xs])
    assert abs(vals.min() + 0.169971) < 1e-5
    assert abs(xs[vals.argmin()] + 0.7518) < 2e-3


def exact_gelu_block(qb: np.ndarray, s: float):
    cache = {}
    g = np.empty(qb.shape, np.float32)
    for idx, c in np.ndenumerate(qb):
        if c not in cache:
            x = to_f32(frac(np.float32(s)) * int(c))
            cache[c] = np.float32(float(gelu_exact_f32(float(x))))
        g[idx] = cache[c]
    return exact_quantize_block(g)


@pytest.mark.parametrize("case", ["random", "extremes"])
def test_gelu_blocks_match_exact_rule(case):
    g = np.random.default_rng(17)
    q = g.integers(-127, 128, size=(64, 64)).astype(np.int8)
    s = np.array([[0.031, 2.4], [0.0004, 0.09]], np.float32)
    if case == "extremes":
        q[:32, :32] = -g.integers(100, 128, size=(32, 32))   # all far-negative: tiny outputs
        s[0, 0] = 0.1
        q[:32, 32:] = 0                                        # all zero codes
        q[32:, :32] = -g.integers(1, 60, size=(32, 32))      # negative side only
        s[1, 0] = 0.02
    qo, so = oracle.gelu(q, s)
    for bi in range(2):
        for bj in range(2):
            sl = (slice(32 * bi, 32 * bi + 32), slice(32 * bj, 32 * bj + 32))
            eq, es = exact_gelu_block(q[sl], s[bi, bj])
            assert so[bi, bj] == np.float32(es), (bi, bj)
            np.testing.assert_array_equal(qo[sl], eq)


def test_zero_scale_block():
    q = np.full((32, 32), 77, np.int8)
    qo, so = oracle.gelu(q, np.zeros((1, 1), np.float32))
    assert so[0, 0] == 0 and not qo.any()
