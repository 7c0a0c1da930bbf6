"""Pins for the oracle's per-block quantization (CPU only).

Method: one binary32 scale per 32x32 block, INT8 codes (Jetfire summary,
one-line summary and "Approach"; block size B = 32).  Reading pinned here:
s = fl(max|x|/127), q = clamp(rne(fl(x/s)), -127, 127), s = 0 gives q = 0.

Each test checks the oracle against something other than itself: the rule
evaluated in exact rational arithmetic, the nearest-code property, closed
forms (power-of-two round trips, ties), and numpy's own bit manipulations.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact import floor_log2, frac, round_half_even, to_f32
from int8_block_quantized_amd import inputs


def exact_quantize_block(blk: np.ndarray):
    """The quantization rule for one block, in exact rationals."""
    vals = [frac(v) for v in blk.ravel()]
    m = max(abs(v) for v in vals)
    s = to_f32(m / 127)
    if s == 0:
        return np.zeros(blk.shape, np.int8), 0.0
    codes = []
    for v in vals:
        r = to_f32(v / s)
        codes.append(max(-127, min(127, round_half_even(r))))
    return np.array(codes, np.int8).reshape(blk.shape), float(s)


def blocks(a):
    R, C = a.shape
    for bi in range(R // 32):
        for bj in range(C // 32):
            yield bi, bj, a[bi * 32:(bi + 1) * 32, bj * 32:(bj + 1) * 32]


def test_matches_exact_rule_64x96_with_outliers():
    x = inputs.activation(100, 0, 64, 96, n_outlier_cols=3, factor=50.0)
    q, s = oracle.quantize(x)
    assert q.shape == (64, 96) and s.shape == (2, 3)
    for bi, bj, blk in blocks(x):
        eq, es = exact_quantize_block(blk)
        assert s[bi, bj] == np.float32(es), (bi, bj)
        np.testing.assert_array_equal(q[bi * 32:(bi + 1) * 32, bj * 32:(bj + 1) * 32], eq)


def test_nearest_code_brute_force_64x64():
    """q is the code n in [-127, 127] minimising |x - s*n| (exactly), except
    where fl(x/s) lands within one ulp of a half-integer (double rounding)."""
    x = inputs.activation(101, 0, 64, 64, n_outlier_cols=2, factor=50.0)
    q, s = oracle.quantize(x)
    exceptions = 0
    for bi, bj, blk in blocks(x):
        sc = frac(s[bi, bj])
        qb = q[bi * 32:(bi + 1) * 32, bj * 32:(bj + 1) * 32]
        for (r, c), v in np.ndenumerate(blk):
            xv = frac(v)
            best = min(range(-127, 128), key=lambda n: (abs(xv - sc * n), n % 2))
            if best != qb[r, c]:
                t = xv / sc
                ulp = Fraction(2) ** -17
                assert abs(abs(t - int(t)) - Fraction(1, 2)) <= ulp
                exceptions += 1
    assert exceptions <= 2


def test_error_bound_and_range():
    x = inputs.activation(102, 0, 256, 256, n_outlier_cols=4, factor=50.0)
    q, s = oracle.quantize(x)
    srep = np.repeat(np.repeat(s.astype(np.float64), 32, 0), 32, 1)
    err = np.abs(x.astype(np.float64) - srep * q.astype(np.float64))
    assert np.all(err <= srep * (0.5 + 2.0 ** -18))
    assert q.min() >= -127 and q.max() <= 127
    # every block reaches +-127 exactly at its max-magnitude element
    for bi, bj, blk in blocks(x):
        qb = q[bi * 32:(bi + 1) * 32, bj * 32:(bj + 1) * 32]
        am = np.abs(blk)
        assert np.all(np.abs(qb[am == am.max()]) == 127)


def test_power_of_two_round_trip_exact():
    """x = 2^e * n with integer |n| <= 127 and a +-127 in every block gives
    s = 2^e, q = n and s*q = x exactly."""
    g = np.random.default_rng(7)
    n = g.integers(-127, 128, size=(96, 64)).astype(np.int8)
    exps = np.array([[-20, 3], [0, -7], [12, -1]])
    x = np.empty(n.shape, np.float32)
    for bi in range(3):
        for bj in range(2):
            sl = (slice(bi * 32, bi * 32 + 32), slice(bj * 32, bj * 32 + 32))
            n[sl][5, 7] = 127 if (bi + bj) % 2 else -127
            x[sl] = np.ldexp(n[sl].astype(np.float32), exps[bi, bj])
    q, s = oracle.quantize(x)
    np.testing.assert_array_equal(q, n)
    np.testing.assert_array_equal(s, np.ldexp(np.ones((3, 2), np.float32), exps))
    np.testing.assert_array_equal(oracle.dequantize(q, s), x)


def test_ties_round_to_even():
    """With s = 1 exactly (block max 127), x = k + 0.5 is an exact tie."""
    x = np.zeros((32, 32), np.float32)
    x[0, 0] = 127.0
    ties = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 125.5, 126.5, -126.5], np.float32)
    x[1, :len(ties)] = ties
    q, s = oracle.quantize(x)
    assert s[0, 0] == 1.0
    np.testing.assert_array_equal(q[1, :len(ties)], [0, 2, 2, 4, 0, -2, -2, 126, 126, -126])


def test_zero_and_underflow_blocks():
    x = np.zeros((32, 128), np.float32)
    x[3, 32 + 4] = np.float32(1e-45)      # max/127 underflows to zero -> s = 0, q = 0
    x[0, 64:96] = np.float32(1e-37)       # subnormal scale, still exact rule
    x[1, 64] = np.float32(-3e-37)
    x[2, 96:128] = np.linspace(-1, 1, 32, dtype=np.float32)
    q, s = oracle.quantize(x)
    assert s[0, 0] == 0 and not q[:, :32].any()
    assert s[0, 1] == 0 and not q[:, 32:64].any()
    eq, es = exact_quantize_block(x[:, 64:96])
    assert s[0, 2] == np.float32(es) and 0 < es < 2.0 ** -126
    np.testing.assert_array_equal(q[:, 64:96], eq)
    eq, es = exact_quantize_block(x[:, 96:128])
    assert s[0, 3] == np.float32(es)
    np.testing.assert_array_equal(q[:, 96:128], eq)


def test_transpose_consistency():
    """32x32 blocks are square, so quantize(X^T) == quantize(X)^T bit for bit:
    the same codes and scales serve the transposed operand of the gradients."""
    x = inputs.activation(103, 0, 128, 96, n_outlier_cols=3, factor=50.0)
    q, s = oracle.quantize(x)
    qt, st = oracle.quantize(np.ascontiguousarray(x.T))
    np.testing.assert_array_equal(qt, q.T)
    np.testing.assert_array_equal(st, s.T)


def test_bf16_input_is_exact_widening():
    x = inputs.activation(104, 0, 64, 64, n_outlier_cols=2, factor=50.0)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    widened = (bits.astype(np.uint32) << 16).view(np.float32)
    qb, sb = oracle.quantize(bits)
    for bi, bj, blk in blocks(widened):
        eq, es = exact_quantize_block(blk)
        assert sb[bi, bj] == np.float32(es)
        np.testing.assert_array_equal(qb[bi * 32:(bi + 1) * 32, bj * 32:(bj + 1) * 32], eq)


def test_requant_is_the_same_rule():
    x = inputs.normal(105, 2, 0, 64, 64, 1e-3)
    q, s = oracle.requant(x)
    for bi, bj, blk in blocks(x):
        eq, es = exact_quantize_block(blk)
        assert s[bi, bj] == np.float32(es)
        np.testing.assert_array_equal(q[bi * 32:(bi + 1) * 32, bj * 32:(bj + 1) * 32], eq)


def test_dequantize_is_blockwise_product():
    g = np.random.default_rng(9)
    q = g.integers(-127, 128, size=(64, 96)).astype(np.int8)
    s = g.random((2, 3)).astype(np.float32)
    ref = (np.repeat(np.repeat(s.astype(np.float64), 32, 0), 32, 1) * q).astype(np.float32)
    np.testing.assert_array_equal(oracle.dequantize(q, s), ref)


def test_bad_shapes_rejected():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((33, 32), np.float32))


def nearest_bf16_exact(v: Fraction) -> Fraction:
    """The bfloat16 value nearest to v (8 significant bits, binary32's
    exponent range, ties to the even significand), in exact rationals."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = max(floor_log2(a), -126)
    ulp = Fraction(2) ** (e - 7)
    return sign * round_half_even(a / ulp) * ulp


def bf16_value(bits: int) -> Fraction:
    return frac(np.array([bits << 16], np.uint32).view(np.float32)[0])


def test_bf16_round_is_nearest_even_exact():
    """The oracle's binary32 -> bfloat16 rounding against the nearest-even
    rule in exact rationals: random values over the whole exponent range,
    subnormals, and every halfway case (and its two binary32 neighbours) on
    a grid of significands and exponents."""
    g = np.random.default_rng(21)
    f = (g.standard_normal(3000) * np.exp2(g.integers(-140, 120, 3000))).astype(np.float32)
    ties = []
    for e in (-133, -126, -20, -1, 0, 1, 7, 60, 126):
        for m in range(0, 128, 9):
            half = np.float32(2.0 ** e * (1 + m / 128) + 2.0 ** (e - 8)) if e >= -126 else np.float32(
                2.0 ** -126 * m / 128 + 2.0 ** (-134))
            ties += [half, -half, np.nextafter(half, np.float32(0)), np.nextafter(half, np.float32(np.inf))]
    f = np.concatenate([f, np.array(ties, np.float32), np.array([0.0, -0.0, 1e-45, -1e-45], np.float32)])
    got = oracle.bf16_round(f)
    for x, b in zip(f, got):
        assert bf16_value(int(b)) == nearest_bf16_exact(frac(x)), (x, hex(b))


def test_bf16_round_matches_torch_and_overflows():
    """Library cross-check (torch's CPU conversion rounds to nearest even)
    on 2^20 random values, plus the overflow edge: the largest binary32
    rounds up to infinity, the largest bfloat16 stays."""
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(22)
    f = (g.standard_normal(1 << 20) * np.exp2(g.integers(-140, 127, 1 << 20))).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.bf16_round(f), ref)
    big = np.array([np.finfo(np.float32).max, 3.3895314e38, -np.finfo(np.float32).max], np.float32)
    assert list(oracle.bf16_round(big)) == [0x7F80, 0x7F7F, 0xFF80]


def test_dequantize_bf16_rounds_the_binary32_product():
    g = np.random.default_rng(23)
    q = g.integers(-127, 128, size=(64, 96)).astype(np.int8)
    s = (g.random((2, 3)) * np.exp2(g.integers(-30, 30, (2, 3)))).astype(np.float32)
    s[1, 2] = 0.0
    y32 = (np.repeat(np.repeat(s.astype(np.float64), 32, 0), 32, 1) * q).astype(np.float32)
    got = oracle.dequantize_bf16(q, s)
    want = np.array([int(b) for b in oracle.bf16_round(y32)], np.uint16).reshape(q.shape)
    np.testing.assert_array_equal(got, want)
    for x, b in zip(y32.ravel()[::37], got.ravel()[::37]):
        assert bf16_value(int(b)) == nearest_bf16_exact(frac(x))
    assert not (got[32:, 64:] & 0x7FFF).any()   # a zero scale gives zeros (negative codes: -0)
