"""Pins for the oracle's INT8 GELU backward (CPU only).

Method: every operator of the INT8 data flow, the backward pass included,
reads and writes INT8 tensors with per-block scales (Jetfire summary,
"Approach").  Reading pinned here: dy = fl(s_dy*q_dy), x = fl(s_x*q_x),
GELU'(x) = Phi(x) + x*phi(x) evaluated in binary64 and rounded once to
binary32, y = fl(dy * GELU'(x)), then per-block requantization.

References: mpmath at 50 significant digits, closed forms of the
derivative, a finite difference of the oracle's own forward GELU (a
different formula), and the exact quantization rule.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle
from exact import frac, to_f32
from test_oracle_quant import exact_quantize_block

mpmath.mp.dps = 50


def gelu_grad_exact_f32(x: float) -> Fraction:
    """Correctly rounded binary32 of Phi(x) + x*phi(x)."""
    xm = mpmath.mpf(float(x))
    d = mpmath.erfc(-xm / mpmath.sqrt(2)) / 2 + xm * mpmath.exp(-xm * xm / 2) / mpmath.sqrt(2 * mpmath.pi)
    if d == 0:
        return Fraction(0)
    sign, man, exp, _ = d._mpf_
    return to_f32((-1) ** sign * Fraction(int(man)) * Fraction(2) ** int(exp))


def sample_points():
    g = np.random.default_rng(7)
    pts = [0.0, -0.0, 1e-30, -1e-30, 0.5, -0.5, -0.7518, -0.75179, 1.0, -1.0, 2.0, -2.0, 3.0, -3.0,
           5.5, -5.5, 8.0, -8.0, 12.0, -12.0, 40.0, -40.0, 127.0, -127.0]
    pts += list(g.standard_normal(300).astype(np.float32) * 3)
    s = np.float32(0.0273)
    pts += [float(s * np.float32(c)) for c in range(-128, 128)]
    return [float(np.float32(p)) for p in pts]


def test_gelu_grad_value_is_correctly_rounded_binary32():
    for x in sample_points():
        assert frac(oracle.gelu_grad_value(x)) == gelu_grad_exact_f32(x), x


def test_closed_forms():
    assert oracle.gelu_grad_value(0.0) == 0.5
    # GELU'(x) + GELU'(-x) = 1 (Phi(x) + Phi(-x) = 1, x phi(x) is odd)
    for x in [0.1, 0.4, 0.7518, 1.3, 2.5, 4.0, 6.0]:
        assert abs(oracle.gelu_grad_value(x) + oracle.gelu_grad_value(-x) - 1.0) <= 2 * 2.0 ** -24, x
    # limits: 1 for large x, 0 from below for very negative x
    for x in [9.0, 20.0, 1e6]:
        assert oracle.gelu_grad_value(x) == 1.0
    for x in [-9.0, -20.0]:
        v = oracle.gelu_grad_value(x)
        assert v <= 0.0 and abs(v) < 1e-16
    # the derivative vanishes where GELU has its minimum, near x = -0.7518
    xs = np.linspace(-0.80, -0.70, 2001, dtype=np.float32)
    vals = np.array([oracle.gelu_grad_value(float(x)) for x in xs])
    cross = xs[np.argmin(np.abs(vals))]
    assert abs(cross + 0.75179) < 1e-4


def test_matches_finite_difference_of_forward_gelu():
    # central difference of x*Phi(x) (the forward oracle, a different formula)
    for x in [-3.0, -1.7, -0.75, -0.2, 0.0, 0.3, 1.1, 2.4, 4.0]:
        h = 2.0 ** -8
        fd = (oracle.gelu_value(x + h) - oracle.gelu_value(x - h)) / (2 * h)
        assert abs(fd - oracle.gelu_grad_value(x)) < 2e-4, x


def exact_gelu_bwd_block(qdy, sdy, qx, sx):
    y = np.empty(qx.shape, np.float32)
    cache = {}
    for idx, c in np.ndenumerate(qx):
        if c not in cache:
            x = to_f32(frac(np.float32(sx)) * int(c))
            cache[c] = gelu_grad_exact_f32(float(x))
        dy = to_f32(frac(np.float32(sdy)) * int(qdy[idx]))
        y[idx] = np.float32(float(to_f32(dy * cache[c])))
    return exact_quantize_block(y)


@pytest.mark.parametrize("case", ["random", "extremes"])
def test_gelu_bwd_blocks_match_exact_rule(case):
    g = np.random.default_rng(31)
    qx = g.integers(-127, 128, size=(64, 64)).astype(np.int8)
    qdy = g.integers(-127, 128, size=(64, 64)).astype(np.int8)
    sx = np.array([[0.031, 2.4], [0.0004, 0.09]], np.float32)
    sdy = np.array([[1e-3, 0.5], [2e-5, 7.0]], np.float32)
    if case == "extremes":
        qx[:32, :32] = -g.integers(100, 128, size=(32, 32))   # far-negative x: tiny derivative
        sx[0, 0] = 0.1
        qx[:32, 32:] = 0                                        # x = 0: derivative 1/2
        qdy[32:, :32] = 0                                       # zero gradient block
        qx[32:, 32:] = -128                                     # the byte outside the code range
    qo, so = oracle.gelu_bwd(qdy, sdy, qx, sx)
    for bi in range(2):
        for bj in range(2):
            sl = (slice(32 * bi, 32 * bi + 32), slice(32 * bj, 32 * bj + 32))
            eq, es = exact_gelu_bwd_block(qdy[sl], sdy[bi, bj], qx[sl], sx[bi, bj])
            assert so[bi, bj] == np.float32(es), (case, bi, bj)
            np.testing.assert_array_equal(qo[sl], eq)


def test_zero_scales():
    q = np.full((32, 64), 77, np.int8)
    qo, so = oracle.gelu_bwd(q, np.array([[0.0, 1.0]], np.float32), q, np.array([[1.0, 0.0]], np.float32))
    assert so[0, 0] == 0 and not qo[:, :32].any()
    # x = 0 everywhere in the second block: y = dy / 2, so the block is the halved codes' requantization
    assert so[0, 1] == np.float32(np.float32(77.0) * np.float32(0.5)) / np.float32(127.0)
    assert np.all(qo[:, 32:] == 127)


def test_bad_shapes_rejected():
    with pytest.raises(ValueError):
        oracle.gelu_bwd(np.zeros((32, 64), np.int8), np.ones((1, 2), np.float32),
                        np.zeros((32, 32), np.int8), np.ones((1, 1), np.float32))
