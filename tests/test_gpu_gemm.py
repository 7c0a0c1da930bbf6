"""GPU parity: jf_gemm_i8_blockscaled vs the CPU oracle.

Bars: int32 partials bit-exact; binary32 output within 1e-5 of the oracle
(per element against sum_k |sigma_k P_k|, and normwise); INT8 output codes
within 1 LSB on at most 0.01% of elements with scales within 1e-6 relative.
Cases: all four transpose combinations, both output kinds, shapes that span
several workgroup tiles with ragged tails in M, N and K, strided views,
K = 0, ties and overflowing reciprocals in the requantizing epilogue, the
tiny forward workload, and the GPT2-base / GPT2-medium MLP workloads at full
size on sampled output blocks.  Whole-output checks of the main tile and the
hidden-4096 GEMMs are in test_gpu_gemm_full.py.
"""
import ctypes
import itertools

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, assert_f32_close, assert_requant_close, block_abs_terms, dev, host, note
from int8_block_quantized_amd import inputs
from int8_block_quantized_amd import jetfire as jf

pytestmark = pytest.mark.gpu
COMBOS = list(itertools.product((0, 1), (0, 1)))


def stored(logical, trans):
    return np.ascontiguousarray(logical.T) if trans else logical


def logical(stored_arr, trans):
    return np.ascontiguousarray(stored_arr.T) if trans else stored_arr


def random_operands(seed, M, N, K, ta, tb):
    A = inputs.codes(300 + seed, 0, 0, M, K)
    B = inputs.codes(300 + seed, 0, 1, K, N)
    sA = inputs.scales(300 + seed, 0, 2, M // 32, K // 32)
    sB = inputs.scales(300 + seed, 0, 3, K // 32, N // 32)
    return stored(A, ta), stored(sA, ta), stored(B, tb), stored(sB, tb), (A, sA, B, sB)


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_int32_partials_bit_exact(ta, tb):
    """K = 32 and unit scales: the binary32 output is the int32 partial."""
    M, N, K = 96, 160, 32
    A, _, B, _, (Al, _, Bl, _) = random_operands(1, M, N, K, ta, tb)
    ones_a = np.ones((K // 32, M // 32) if ta else (M // 32, K // 32), np.float32)
    ones_b = np.ones((N // 32, K // 32) if tb else (K // 32, N // 32), np.float32)
    C = host(jf.gemm_i8_blockscaled(dev(A), dev(ones_a), dev(B), dev(ones_b), ta, tb, out="f32"))
    ref = Al.astype(np.int64) @ Bl.astype(np.int64)
    np.testing.assert_array_equal(C.astype(np.int64), ref)
    for I, J in [(0, 0), (2, 4), (1, 3)]:
        P = oracle.gemm_partial(A, B, I, J, 0, ta=ta, tb=tb)
        np.testing.assert_array_equal(C[32 * I:32 * I + 32, 32 * J:32 * J + 32].astype(np.int64), P)


@pytest.mark.parametrize("ta,tb", COMBOS)
@pytest.mark.parametrize("shape", [(160, 224, 96), (256, 128, 320), (32, 32, 32)])
def test_random_codes_full_compare(ta, tb, shape):
    M, N, K = shape
    A, sA, B, sB, (Al, sAl, Bl, sBl) = random_operands(2 + sum(shape) // 32, M, N, K, ta, tb)
    dA, dsA, dB, dsB = dev(A), dev(sA), dev(B), dev(sB)
    C = host(jf.gemm_i8_blockscaled(dA, dsA, dB, dsB, ta, tb, out="f32"))
    q, s = jf.gemm_i8_blockscaled(dA, dsA, dB, dsB, ta, tb, out="i8")
    Cref = oracle.gemm_f32(A, sA, B, sB, ta=ta, tb=tb)
    qref, sref = oracle.gemm_i8(A, sA, B, sB, ta=ta, tb=tb)
    for I in range(M // 32):
        for J in range(N // 32):
            sl = (slice(32 * I, 32 * I + 32), slice(32 * J, 32 * J + 32))
            assert_f32_close(C[sl], Cref[sl], block_abs_terms(Al, sAl, Bl, sBl, I, J), f"block {I},{J}")
    exact = float((C == Cref).mean())
    frac, srel = assert_requant_close(host(q), host(s), qref, sref, "i8 out")
    note(f"gemm {shape} tA={ta} tB={tb}: f32 bit-exact {exact:.4f}, i8 code diffs {frac:.2e}, scale rel {srel:.1e}")


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_strided_views(ta, tb):
    M, N, K = 64, 96, 128
    A, sA, B, sB, _ = random_operands(9, M, N, K, ta, tb)
    bigA = torch.zeros((A.shape[0], A.shape[1] + 48), dtype=torch.int8, device=DEV)
    bigA[:, 16:16 + A.shape[1]] = dev(A)
    bigB = torch.zeros((B.shape[0], B.shape[1] + 32), dtype=torch.int8, device=DEV)
    bigB[:, :B.shape[1]] = dev(B)
    cbig = torch.full((M, N + 64), -5.0, dtype=torch.float32, device=DEV)
    jf.gemm_i8_blockscaled(bigA[:, 16:16 + A.shape[1]], dev(sA), bigB[:, :B.shape[1]], dev(sB), ta, tb,
                           out="f32", c=cbig[:, 32:32 + N])
    got = host(cbig)
    ref = oracle.gemm_f32(A, sA, B, sB, ta=ta, tb=tb)
    np.testing.assert_array_equal(got[:, 32:32 + N], ref)
    assert np.all(got[:, :32] == -5.0) and np.all(got[:, 32 + N:] == -5.0)


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_wide_leading_dimension(ta, tb):
    """Leading dimensions of 2^24 + 64 bytes: per-lane load offsets no longer
    fit in 32 bits, which selects the kernels' 64-bit address path."""
    M, N, K = 64, 96, 128
    A, sA, B, sB, _ = random_operands(10, M, N, K, ta, tb)
    ld = (1 << 24) + 64
    note(f"wide ld: ta={ta} tb={tb}, operand buffers of {A.shape[0] * ld / 2**20:.0f} and "
         f"{B.shape[0] * ld / 2**20:.0f} MiB")
    bigA = torch.empty((A.shape[0], ld), dtype=torch.int8, device=DEV)
    bigA[:, :A.shape[1]] = dev(A)
    bigB = torch.empty((B.shape[0], ld), dtype=torch.int8, device=DEV)
    bigB[:, ld - B.shape[1]:] = dev(B)
    got = host(jf.gemm_i8_blockscaled(bigA[:, :A.shape[1]], dev(sA), bigB[:, ld - B.shape[1]:], dev(sB),
                                      ta, tb, out="f32"))
    del bigA, bigB
    np.testing.assert_array_equal(got, oracle.gemm_f32(A, sA, B, sB, ta=ta, tb=tb))


def test_k_zero_writes_zeros():
    M, N = 64, 96
    dummy = torch.zeros(64, dtype=torch.int8, device=DEV)
    fdummy = torch.ones(16, dtype=torch.float32, device=DEV)
    c = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
    q = torch.full((M, N), 7, dtype=torch.int8, device=DEV)
    s = torch.full((M // 32, N // 32), 7.0, dtype=torch.float32, device=DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = jf.lib.jf_gemm_i8_blockscaled(0, 0, M, N, 0, p(dummy), 0, p(fdummy), p(dummy), N, p(fdummy),
                                       jf.JF_OUT_F32, p(c), N, None, st)
    assert rc == jf.JF_OK
    rc = jf.lib.jf_gemm_i8_blockscaled(0, 0, M, N, 0, p(dummy), 0, p(fdummy), p(dummy), N, p(fdummy),
                                       jf.JF_OUT_I8, p(q), N, p(s), st)
    assert rc == jf.JF_OK
    assert not host(c).any() and not host(q).any() and not host(s).any()


def quantized(wl, name, cache):
    if name not in cache:
        x = wl.make(name)
        q, s = jf.quantize_block(dev(x))
        oq, os_ = oracle.quantize(x)
        cache[name] = (q, s, oq, os_)
    return cache[name]


def sample_blocks(M, N, n, seed):
    g = np.random.default_rng(seed)
    nbM, nbN = M // 32, N // 32
    blks = {(0, 0), (nbM - 1, nbN - 1), (0, nbN - 1), (nbM - 1, 0)}
    while len(blks) < n:
        blks.add((int(g.integers(nbM)), int(g.integers(nbN))))
    return sorted(blks)


def check_workload_gemms(wl, n_blocks, f32_labels=()):
    cache = {}
    for (label, ta, tb, M, N, K, an, bn) in wl.gemms():
        qa, sa, oqa, osa = quantized(wl, an, cache)
        qb, sb, oqb, osb = quantized(wl, bn, cache)
        note(f"{wl.name}: {label} (M={M} N={N} K={K} tA={ta} tB={tb})")
        q, s = jf.gemm_i8_blockscaled(qa, sa, qb, sb, ta, tb, out="i8")
        blks = sample_blocks(M, N, n_blocks, M + N + K)
        qh, sh = host(q), host(s)
        oq, os_ = oracle.gemm_i8_blocks(oqa, osa, oqb, osb, blks, ta=ta, tb=tb)
        gq = np.stack([qh[32 * I:32 * I + 32, 32 * J:32 * J + 32] for I, J in blks])
        gs = np.array([sh[I, J] for I, J in blks])
        frac, srel = assert_requant_close(gq, gs, oq, os_, label)
        msg = f"  i8: code diffs {frac:.2e} scale rel {srel:.1e}"
        if label in f32_labels:
            C = host(jf.gemm_i8_blockscaled(qa, sa, qb, sb, ta, tb, out="f32"))
            oc = oracle.gemm_f32_blocks(oqa, osa, oqb, osb, blks, ta=ta, tb=tb)
            Al, sAl = logical(oqa, ta), logical(osa, ta)
            Bl, sBl = logical(oqb, tb), logical(osb, tb)
            ex = []
            for n_, (I, J) in enumerate(blks):
                gc = C[32 * I:32 * I + 32, 32 * J:32 * J + 32]
                ex.append(assert_f32_close(gc, oc[n_], block_abs_terms(Al, sAl, Bl, sBl, I, J), f"{label} {I},{J}"))
            msg += f"; f32 bit-exact {np.mean(ex):.4f}"
            del C
        note(msg)
        del q, s
    # the quantized operands themselves are bit-exact
    for name, (q, s, oq, os_) in cache.items():
        np.testing.assert_array_equal(host(s), os_, err_msg=f"{name} scales")
        np.testing.assert_array_equal(host(q), oq, err_msg=f"{name} codes")


def test_tiny_forward_workload():
    wl = inputs.tiny_forward()
    x, w = wl.make("X"), wl.make("W")
    qx, sx = jf.quantize_block(dev(x))
    qw, sw = jf.quantize_block(dev(w))
    oqx, osx = oracle.quantize(x)
    oqw, osw = oracle.quantize(w)
    C = host(jf.gemm_i8_blockscaled(qx, sx, qw, sw, out="f32"))
    np.testing.assert_array_equal(C, oracle.gemm_f32(oqx, osx, oqw, osw))
    q, s = jf.gemm_i8_blockscaled(qx, sx, qw, sw, out="i8")
    oq, os_ = oracle.gemm_i8(oqx, osx, oqw, osw)
    assert_requant_close(host(q), host(s), oq, os_, "tiny i8")
    check_workload_gemms(wl, 64, f32_labels=("fc.fwd", "fc.dgrad", "fc.wgrad"))


def test_gpt2_base_linear_full_size():
    check_workload_gemms(inputs.gpt2_base_linear(), 24, f32_labels=("fc.fwd", "fc.dgrad", "fc.wgrad"))


@pytest.mark.parametrize("ta,tb", COMBOS)
@pytest.mark.parametrize("scale", [1.0, 1e-20])
def test_requant_epilogue_ties_and_tiny_scales(ta, tb, scale):
    """INT8 output where the codes sit exactly on half-integers: every column
    of B holds two ones, so acc = a + a' (an integer, |acc| <= 254) and each
    output block's maximum is 254, so s = 2 and every odd acc is a tie that
    only the IEEE quotient decides (round half to even).  With scales of
    1e-20 the products are subnormal and fl(1/s) overflows, so every element
    takes the quotient path.  Codes and scales must match the oracle
    exactly."""
    M, N, K = 64, 96, 64
    g = np.random.default_rng(77)
    A = g.integers(-127, 128, size=(M, K)).astype(np.int8)
    B = np.zeros((K, N), np.int8)
    t1 = g.integers(0, K, size=N)
    t2 = (t1 + 1 + g.integers(0, K - 1, size=N)) % K
    B[t1, np.arange(N)] = 1
    B[t2, np.arange(N)] = 1
    for I in range(M // 32):
        for J in range(N // 32):
            A[32 * I, t1[32 * J]] = 127
            A[32 * I, t2[32 * J]] = 127
    sA = np.full((M // 32, K // 32), scale, np.float32)
    sB = np.full((K // 32, N // 32), scale, np.float32)
    As, sAs, Bs, sBs = stored(A, ta), stored(sA, ta), stored(B, tb), stored(sB, tb)
    q, s = jf.gemm_i8_blockscaled(dev(As), dev(sAs), dev(Bs), dev(sBs), ta, tb, out="i8")
    oq, os_ = oracle.gemm_i8(As, sAs, Bs, sBs, ta=ta, tb=tb)
    np.testing.assert_array_equal(host(s), os_)
    np.testing.assert_array_equal(host(q), oq)
    if scale == 1.0:
        assert np.all(os_ == 2.0)
        acc = A.astype(np.int64) @ B.astype(np.int64)
        assert (acc % 2 != 0).mean() > 0.3, "too few ties to exercise the rule"
