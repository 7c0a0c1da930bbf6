"""Pins for the oracle's block-scaled INT8 GEMM (CPU only).

Method: linear operators, the weight gradient included, run on INT8 codes
with per-block (32x32) scales (Jetfire summary, "Approach").  Reading pinned
here: for each output element, k-blocks in ascending order, the exact int32
partial P of a 32-deep k-block, sigma = fl(sA*sB), acc = fmaf(sigma, P, acc).

Independent references: numpy int64 matmul (exact integers), numpy float64
matmul of blockwise-dequantized operands with a derived rounding bound, and
the fused sequence replayed in exact rationals.
"""
import itertools

import numpy as np
import pytest

import oracle
from exact import frac, to_f32
from test_oracle_quant import exact_quantize_block

COMBOS = list(itertools.product((0, 1), (0, 1)))


def stored(logical: np.ndarray, trans: int) -> np.ndarray:
    return np.ascontiguousarray(logical.T) if trans else logical


def rand_codes(g, shape):
    return g.integers(-127, 128, size=shape).astype(np.int8)


def rand_scales(g, shape):
    # spread over several decades so a scale taken from the wrong block shows
    return (g.random(shape) * 1.5 + 0.5) * 10.0 ** g.integers(-3, 2, size=shape)


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_unit_scale_equals_integer_matmul(ta, tb):
    """Unit scales and K <= 512 keep every partial sum below 2^24, so the
    binary32 result equals the exact integer product."""
    g = np.random.default_rng(11 + 2 * ta + tb)
    M, N, K = 64, 96, 160
    A, B = rand_codes(g, (M, K)), rand_codes(g, (K, N))
    C = oracle.gemm_f32(stored(A, ta), np.ones((M // 32, K // 32) if not ta else (K // 32, M // 32), np.float32),
                        stored(B, tb), np.ones((K // 32, N // 32) if not tb else (N // 32, K // 32), np.float32),
                        ta=ta, tb=tb)
    ref = A.astype(np.int64) @ B.astype(np.int64)
    np.testing.assert_array_equal(C.astype(np.int64), ref)


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_int32_partials(ta, tb):
    g = np.random.default_rng(21 + 2 * ta + tb)
    M, N, K = 64, 96, 128
    A, B = rand_codes(g, (M, K)), rand_codes(g, (K, N))
    for (I, J, kb) in [(0, 0, 0), (1, 2, 3), (1, 0, 2), (0, 2, 1)]:
        P = oracle.gemm_partial(stored(A, ta), stored(B, tb), I, J, kb, ta=ta, tb=tb)
        ref = A[32 * I:32 * I + 32, 32 * kb:32 * kb + 32].astype(np.int64) @ \
            B[32 * kb:32 * kb + 32, 32 * J:32 * J + 32].astype(np.int64)
        np.testing.assert_array_equal(P, ref)
    # extreme partials: all -127 x 127 gives -32*127^2, inside int32
    A8 = np.full((32, 32), -127, np.int8)
    B8 = np.full((32, 32), 127, np.int8)
    assert oracle.gemm_partial(A8, B8, 0, 0, 0).min() == -32 * 127 * 127


def blockwise(s_log: np.ndarray) -> np.ndarray:
    return np.repeat(np.repeat(s_log.astype(np.float64), 32, 0), 32, 1)


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_scaled_against_float64_matmul(ta, tb):
    """Against float64 matmul of the dequantized operands, within the
    rounding bound of a K/32-term fused chain with a rounded scale product:
    |err| <= (2 K/32 + 2) u sum_k |sigma_k P_k|, u = 2^-24."""
    g = np.random.default_rng(31 + 2 * ta + tb)
    M, N, K = 96, 64, 256
    A, B = rand_codes(g, (M, K)), rand_codes(g, (K, N))
    sA_log = rand_scales(g, (M // 32, K // 32)).astype(np.float32)
    sB_log = rand_scales(g, (K // 32, N // 32)).astype(np.float32)
    C = oracle.gemm_f32(stored(A, ta), stored(sA_log, ta), stored(B, tb), stored(sB_log, tb), ta=ta, tb=tb)
    Ad = A * blockwise(sA_log)
    Bd = B * blockwise(sB_log)
    ref = Ad @ Bd
    absum = np.zeros((M, N))
    for kb in range(K // 32):
        ks = slice(32 * kb, 32 * kb + 32)
        absum += np.abs(Ad[:, ks] @ Bd[ks, :])
    nk = K // 32
    bound = (2 * nk + 2) * 2.0 ** -24 * absum + 1e-30
    err = np.abs(C.astype(np.float64) - ref)
    assert np.all(err <= bound), float((err / bound).max())
    # a scale read from the transposed grid would be far outside the bound
    wrong = (A * blockwise(sA_log)) @ (B * blockwise(np.ascontiguousarray(sB_log[::-1])))
    assert np.any(np.abs(wrong - ref) > 1e3 * bound)


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_fused_sequence_in_exact_rationals(ta, tb):
    """Replays acc <- RN32(RN32(sA*sB) * P + acc), k-blocks ascending, in
    exact arithmetic: the oracle must agree bit for bit."""
    g = np.random.default_rng(41 + 2 * ta + tb)
    M, N, K = 64, 32, 96
    A, B = rand_codes(g, (M, K)), rand_codes(g, (K, N))
    sA_log = rand_scales(g, (M // 32, K // 32)).astype(np.float32)
    sB_log = rand_scales(g, (K // 32, N // 32)).astype(np.float32)
    C = oracle.gemm_f32(stored(A, ta), stored(sA_log, ta), stored(B, tb), stored(sB_log, tb), ta=ta, tb=tb)
    parts = [A[:, 32 * kb:32 * kb + 32].astype(np.int64) @ B[32 * kb:32 * kb + 32, :].astype(np.int64)
             for kb in range(K // 32)]
    for i in range(M):
        for j in range(N):
            acc = frac(0.0)
            for kb in range(K // 32):
                sigma = to_f32(frac(sA_log[i // 32, kb]) * frac(sB_log[kb, j // 32]))
                acc = to_f32(sigma * int(parts[kb][i, j]) + acc)
            assert frac(C[i, j]) == acc, (i, j)


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_transposed_storage_gives_identical_bits(ta, tb):
    g = np.random.default_rng(51 + 2 * ta + tb)
    M, N, K = 64, 96, 128
    A, B = rand_codes(g, (M, K)), rand_codes(g, (K, N))
    sA_log = rand_scales(g, (M // 32, K // 32)).astype(np.float32)
    sB_log = rand_scales(g, (K // 32, N // 32)).astype(np.float32)
    C0 = oracle.gemm_f32(A, sA_log, B, sB_log)
    C1 = oracle.gemm_f32(stored(A, ta), stored(sA_log, ta), stored(B, tb), stored(sB_log, tb), ta=ta, tb=tb)
    np.testing.assert_array_equal(C0, C1)


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_int8_output_is_blockwise_requant(ta, tb):
    g = np.random.default_rng(61 + 2 * ta + tb)
    M, N, K = 64, 96, 128
    A, B = rand_codes(g, (M, K)), rand_codes(g, (K, N))
    sA_log = rand_scales(g, (M // 32, K // 32)).astype(np.float32)
    sB_log = rand_scales(g, (K // 32, N // 32)).astype(np.float32)
    args = (stored(A, ta), stored(sA_log, ta), stored(B, tb), stored(sB_log, tb))
    C = oracle.gemm_f32(*args, ta=ta, tb=tb)
    q, s = oracle.gemm_i8(*args, ta=ta, tb=tb)
    for bi in range(M // 32):
        for bj in range(N // 32):
            eq, es = exact_quantize_block(C[32 * bi:32 * bi + 32, 32 * bj:32 * bj + 32])
            assert s[bi, bj] == np.float32(es)
            np.testing.assert_array_equal(q[32 * bi:32 * bi + 32, 32 * bj:32 * bj + 32], eq)
    blks = [(0, 0), (1, 2), (0, 1)]
    fb = oracle.gemm_f32_blocks(*args, blks, ta=ta, tb=tb)
    qb, sb = oracle.gemm_i8_blocks(*args, blks, ta=ta, tb=tb)
    for n, (I, J) in enumerate(blks):
        np.testing.assert_array_equal(fb[n], C[32 * I:32 * I + 32, 32 * J:32 * J + 32])
        np.testing.assert_array_equal(qb[n], q[32 * I:32 * I + 32, 32 * J:32 * J + 32])
        assert sb[n] == s[I, J]


def test_zero_scale_blocks_contribute_nothing():
    g = np.random.default_rng(71)
    A, B = rand_codes(g, (32, 64)), rand_codes(g, (64, 32))
    sA = np.array([[0.0, 2.0]], np.float32)
    sB = np.array([[3.0], [0.5]], np.float32)
    C = oracle.gemm_f32(A, sA, B, sB)
    ref = (A[:, 32:].astype(np.int64) @ B[32:, :].astype(np.int64)).astype(np.float64) * 1.0
    np.testing.assert_array_equal(C.astype(np.float64), ref)


def test_bad_dims_rejected():
    with pytest.raises(ValueError):
        oracle.gemm_f32(np.zeros((32, 64), np.int8), np.ones((1, 2), np.float32),
                        np.zeros((32, 32), np.int8), np.ones((1, 1), np.float32))
