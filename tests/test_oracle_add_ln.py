"""Pins for the oracle's residual add and LayerNorm with INT8 in and out (CPU).

Method: every operator of the data flow reads and writes INT8 with one scale
per 32x32 block (Jetfire summary, one-line summary and "Approach").  The
pages name neither operator; the readings pinned here:
  * add:  z = fl(fl(s_a q_a) + fl(s_b q_b)), then the per-block rule;
  * LayerNorm over each row: x = fl(s q), mean and biased variance of the
    row, y = (x - mean) / sqrt(var + eps) * gamma + beta rounded once to
    binary32, then the per-block rule.

References: the add in exact rationals; LayerNorm from 50-digit mpmath (the
statistics, the square root and y are computed far beyond binary64, then
rounded once); closed forms (a + a = 2a, a + (-a) = 0, a constant row
normalizes to beta, exact scale invariance with eps = 0).
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle
from exact import frac, to_f32
from test_oracle_quant import exact_quantize_block

mpmath.mp.dps = 50


def rand_block_tensor(seed, R, C, scale_range=(-4, 1)):
    g = np.random.default_rng(seed)
    q = g.integers(-127, 128, size=(R, C)).astype(np.int8)
    s = (10.0 ** g.uniform(*scale_range, size=(R // 32, C // 32))).astype(np.float32)
    return q, s


def exact_add(qa, sa, qb, sb):
    R, C = qa.shape
    z = np.empty((R, C), np.float32)
    for (i, j), a in np.ndenumerate(qa):
        xa = to_f32(frac(sa[i // 32, j // 32]) * int(a))
        xb = to_f32(frac(sb[i // 32, j // 32]) * int(qb[i, j]))
        z[i, j] = np.float32(float(to_f32(xa + xb)))
    return z


def quantize_exact(z):
    R, C = z.shape
    q = np.empty((R, C), np.int8)
    s = np.empty((R // 32, C // 32), np.float32)
    for bi in range(R // 32):
        for bj in range(C // 32):
            sl = (slice(32 * bi, 32 * bi + 32), slice(32 * bj, 32 * bj + 32))
            q[sl], s[bi, bj] = exact_quantize_block(z[sl])
    return q, s


@pytest.mark.parametrize("case", ["random", "mixed scales", "zero scales"])
def test_add_matches_exact_rule(case):
    qa, sa = rand_block_tensor(51, 64, 96)
    qb, sb = rand_block_tensor(52, 64, 96, (-1, 2) if case == "mixed scales" else (-4, 1))
    if case == "zero scales":
        sa[0, 0] = 0.0
        sb[1, 2] = 0.0
        sa[1, 1] = sb[1, 1] = 0.0
        qb[0:32, 32:64] = -qa[0:32, 32:64]              # cancels where the scales agree
        sb[0, 1] = sa[0, 1]
    qo, so = oracle.add(qa, sa, qb, sb)
    eq, es = quantize_exact(exact_add(qa, sa, qb, sb))
    np.testing.assert_array_equal(so, es)
    np.testing.assert_array_equal(qo, eq)
    if case == "zero scales":
        assert so[1, 1] == 0 and not qo[32:64, 32:64].any()
        assert so[0, 1] == 0 and not qo[0:32, 32:64].any()


def test_add_closed_forms():
    qa, sa = rand_block_tensor(53, 64, 128)
    # a + a: every value doubles exactly, so the codes are those of the
    # dequantized a and the scales double
    q2, s2 = oracle.add(qa, sa, qa, sa)
    qd, sd = oracle.quantize(oracle.dequantize(qa, sa))
    np.testing.assert_array_equal(q2, qd)
    np.testing.assert_array_equal(s2, sd * np.float32(2))
    # a + (-a) = 0
    qz, sz = oracle.add(qa, sa, -qa, sa)
    assert not qz.any() and not sz.any()
    # commutative (each rounding is of a commutative operation)
    qb, sb = rand_block_tensor(54, 64, 128)
    np.testing.assert_array_equal(oracle.add(qa, sa, qb, sb)[0], oracle.add(qb, sb, qa, sa)[0])


def ln_reference(q, s, gamma, beta, eps):
    """y rounded once to binary32 from a 50-digit evaluation of the rule."""
    R, C = q.shape
    y = np.empty((R, C), np.float32)
    for i in range(R):
        x = [mpmath.mpf(float(np.float32(s[i // 32, j // 32]) * np.float32(q[i, j]))) for j in range(C)]
        m = mpmath.fsum(x) / C
        v = mpmath.fsum([(xj - m) ** 2 for xj in x]) / C
        r = 1 / mpmath.sqrt(v + mpmath.mpf(float(np.float32(eps))))
        for j in range(C):
            yj = (x[j] - m) * r * mpmath.mpf(float(gamma[j])) + mpmath.mpf(float(beta[j]))
            y[i, j] = np.float32(float(to_f32(Fraction(mpmath.nstr(yj, 45, strip_zeros=False)))))
    return y, m


def ln_case(seed, R, C, outliers=True):
    q, s = rand_block_tensor(seed, R, C, (-3, 0))
    g = np.random.default_rng(seed + 1)
    if outliers:
        s[:, 1] *= np.float32(100.0)                    # an outlier block column
    gamma = g.normal(1.0, 0.3, size=C).astype(np.float32)
    beta = g.normal(0.0, 0.2, size=C).astype(np.float32)
    return q, s, gamma, beta


@pytest.mark.parametrize("R,C", [(32, 96), (64, 64)])
def test_layernorm_matches_high_precision(R, C):
    q, s, gamma, beta = ln_case(61 + C, R, C)
    qo, so, mean, rstd = oracle.layernorm(q, s, gamma, beta, 1e-5, stats=True)
    y, _ = ln_reference(q, s, gamma, beta, 1e-5)
    eq, es = quantize_exact(y)
    np.testing.assert_array_equal(so, es)
    np.testing.assert_array_equal(qo, eq)
    # the row statistics themselves, against exact sums of the binary32 values
    x = (s.repeat(32, 0).repeat(32, 1) * q.astype(np.float32)).astype(np.float32)
    for i in range(R):
        m = sum(Fraction(float(v)) for v in x[i]) / C
        assert abs(Fraction(mean[i]) - m) <= abs(m) * Fraction(1, 10 ** 13) + Fraction(1, 10 ** 300)


def test_layernorm_constant_rows_give_beta():
    C = 128
    q = np.full((32, C), 5, np.int8)
    q[7, :] = -3
    s = np.full((1, C // 32), 0.25, np.float32)
    g = np.random.default_rng(63)
    gamma = g.normal(1.0, 0.3, size=C).astype(np.float32)
    beta = g.normal(0.0, 0.2, size=C).astype(np.float32)
    qo, so = oracle.layernorm(q, s, gamma, beta, 1e-5)
    eq, es = oracle.quantize(np.tile(beta, (32, 1)))
    np.testing.assert_array_equal(qo, eq)
    np.testing.assert_array_equal(so, es)


def test_layernorm_exact_scale_invariance_without_eps():
    """With eps = 0, doubling every scale doubles every x exactly, the mean
    exactly, the variance by exactly 4 and the reciprocal root by exactly
    1/2, so the output is bit-identical."""
    q, s, gamma, beta = ln_case(64, 64, 128)
    a = oracle.layernorm(q, s, gamma, beta, 0.0)
    b = oracle.layernorm(q, s * np.float32(2), gamma, beta, 0.0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_layernorm_unit_affine_normalizes():
    """gamma = 1, beta = 0: each dequantized output row has mean ~0 and
    variance ~1, within the output's quantization error (|err| <= s/2)."""
    q, s, _, _ = ln_case(65, 64, 256, outliers=False)
    C = q.shape[1]
    qo, so = oracle.layernorm(q, s, np.ones(C, np.float32), np.zeros(C, np.float32), 1e-5)
    y = oracle.dequantize(qo, so).astype(np.float64)
    half = (so.repeat(32, 0).repeat(32, 1) / 2).astype(np.float64)
    for i in range(q.shape[0]):
        tol = half[i].mean()
        assert abs(y[i].mean()) <= tol + 1e-6
        assert abs((y[i] ** 2).mean() - 1.0) <= 2 * np.sqrt((y[i] ** 2).mean()) * half[i].max() + 1e-4


def test_bad_shapes_rejected():
    with pytest.raises(ValueError):
        oracle.add(np.zeros((32, 64), np.int8), np.ones((1, 2), np.float32),
                   np.zeros((32, 32), np.int8), np.ones((1, 1), np.float32))
    with pytest.raises(ValueError):
        oracle.layernorm(np.zeros((32, 64), np.int8), np.ones((1, 2), np.float32),
                         np.ones(32, np.float32), np.zeros(64, np.float32))
