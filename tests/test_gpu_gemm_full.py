"""GPU parity of the block-scaled GEMM over whole outputs and at full size.

1. Main tile, every element.  Grids of at least 512 tiles of 128 x 256 run the
   main tile; a 4128 x 4192 output (33 x 17 tiles) has a ragged last tile row
   (one of four block rows) and tile column (three of eight block columns).
   K = 256 (two-k-block stages) and K = 288 (odd k-block count: one-k-block
   stages), all four transposes, random codes and scales: every element of
   the binary32 and INT8 outputs against the oracle.  Outputs are prefilled
   (NaN, a code pattern) so an unwritten block cannot pass.
2. Hidden-4096 GEMMs, every 32nd block row.  The twelve GEMMs of the
   8192-token block (QKV, out-projection, FC1, FC2; forward, activation
   gradient, weight gradient) at full size on their workload's data, in the
   launch configuration the benchmark times: every 32nd output block row
   (offset per GEMM) against the oracle, binary32 and INT8; the observed
   difference rates are printed.
3. Hidden-4096 GEMMs, every element.  Codes in [-2, 2] and power-of-two scales
   in {1/2, 1, 2}: every partial P, product sigma * P and running sum is then
   an exact binary32 value (multiples of 1/4 below 2^18), so the output is
   the exact sum over k-blocks of sigma * P in any order.  The expected value
   is the float64 product of the dequantized operands (exact for the same
   reason), and the expected INT8 output is the oracle's per-block
   requantization of it.  A skipped, duplicated or misplaced tile, a wrong
   scale index or a stage read before it landed fails here on any block.
4. The 256 x 256 tile of the gradient layouts on a ragged 8224 x 4192 grid:
   every element with the exact construction, the edge blocks against the
   oracle with real codes and scales.
5. 64-bit load offsets on the two large tiles: one operand with a leading
   dimension of 2^23 + 64 bytes, every element with the exact construction.
6. Shapes on both sides of every tile-selection switch (grid sizes, the
   256 x 256 tile's work threshold, odd k-block counts), and 24 seeded random
   small shapes in all layouts: every element with the exact construction.
7. The GPT2-base linear (4096 tokens, 768 -> 3072) and the GPT2-medium MLP
   (8192 tokens, 1024 -> 4096 -> 1024): every GEMM on its workload's data,
   every element of both outputs against the oracle (grids of fewer than
   512 main tiles run the 64 x 128 tile, the others the 128 x 256 one).

The binary32 bar is |gpu - oracle| <= 1e-5 * sum_k |sigma_k P_k| per element
and 1e-5 normwise; the bound is evaluated on the blocks that differ (none is
expected: the kernel's arithmetic is the oracle's, so outputs are bit-exact).
INT8: at most 1 LSB on at most 0.01% of elements, scales within 1e-6.
"""
import itertools
import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, assert_f32_close, assert_requant_close, block_abs_terms, dev, host, note
from int8_block_quantized_amd import inputs
from int8_block_quantized_amd import jetfire as jf

pytestmark = pytest.mark.gpu
COMBOS = list(itertools.product((0, 1), (0, 1)))


def stored(a, trans):
    return np.ascontiguousarray(a.T) if trans else a


def logical(a, trans):
    return np.ascontiguousarray(a.T) if trans else a


def check_f32(got, ref, A, sA, B, sB, ta, tb, blocks_of_rows, what):
    """Bit-exact fraction, and the 1e-5 bars on every block that differs.
    got/ref: the compared rows (2-D); blocks_of_rows maps a row-block index
    of got to the output block row I."""
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    assert not np.isnan(got).any(), f"{what}: unwritten (NaN) outputs"
    diff = got != ref
    if diff.any():
        Al, sAl, Bl, sBl = logical(A, ta), logical(sA, ta), logical(B, tb), logical(sB, tb)
        rb, cb = np.nonzero(diff.reshape(diff.shape[0] // 32, 32, diff.shape[1] // 32, 32).any(axis=(1, 3)))
        for r, c in zip(rb, cb):
            sl = (slice(32 * r, 32 * r + 32), slice(32 * c, 32 * c + 32))
            assert_f32_close(got[sl], ref[sl], block_abs_terms(Al, sAl, Bl, sBl, blocks_of_rows(r), c),
                             f"{what} block {blocks_of_rows(r)},{c}")
        nr = np.linalg.norm(ref.astype(np.float64))
        assert np.linalg.norm((got - ref).astype(np.float64)) <= 1e-5 * nr, f"{what}: normwise bound"
    return 1.0 - float(diff.mean())


def run_gemm(qa, sa, qb, sb, ta, tb, M, N):
    """Both output kinds, into prefilled buffers."""
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    jf.gemm_i8_blockscaled(qa, sa, qb, sb, ta, tb, out="f32", c=c)
    q = torch.full((M, N), 0x55, dtype=torch.int8, device=DEV)
    s = torch.full((M // 32, N // 32), float("nan"), dtype=torch.float32, device=DEV)
    jf.gemm_i8_blockscaled(qa, sa, qb, sb, ta, tb, out="i8", c=q, sc=s)
    return c, q, s


@pytest.mark.parametrize("ta,tb", COMBOS)
@pytest.mark.parametrize("K", [256, 288])
def test_main_tile_full_output(ta, tb, K):
    M, N = 4128, 4192
    seed = 700 + K // 32 + 2 * ta + tb
    A = stored(inputs.codes(seed, 0, 0, M, K), ta)
    B = stored(inputs.codes(seed, 0, 1, K, N), tb)
    sA = stored(inputs.scales(seed, 0, 2, M // 32, K // 32), ta)
    sB = stored(inputs.scales(seed, 0, 3, K // 32, N // 32), tb)
    note(f"main tile full: {M}x{N}x{K} tA={ta} tB={tb}")
    c, q, s = run_gemm(dev(A), dev(sA), dev(B), dev(sB), ta, tb, M, N)
    gc, gq, gs = host(c), host(q), host(s)
    ref = oracle.gemm_f32(A, sA, B, sB, ta=ta, tb=tb)
    exact = check_f32(gc, ref, A, sA, B, sB, ta, tb, lambda r: r, "main tile f32")
    # the oracle's INT8 output is the per-block requantization of its binary32 output
    rq, rs = oracle.requant(ref)
    frac, srel = assert_requant_close(gq, gs, rq, rs, "main tile i8")
    note(f"  every element: f32 bit-exact {exact:.6f}, i8 code diffs {frac:.2e}, scale rel {srel:.1e}")


_CACHE = {}


def quantized(wl, name):
    key = (wl.wid, name)
    if key not in _CACHE:
        if len(_CACHE) > 6:
            _CACHE.clear()
        x = wl.make(name)
        q, s = jf.quantize_block(dev(x))
        oq, os_ = oracle.quantize(x)
        np.testing.assert_array_equal(host(q), oq, err_msg=f"{name} codes")
        np.testing.assert_array_equal(host(s), os_, err_msg=f"{name} scales")
        _CACHE[key] = (q, s, oq, os_)
    return _CACHE[key]


H4096 = {g[0]: g for g in inputs.hidden4096_block().gemms()}


@pytest.mark.parametrize("label", list(H4096))
def test_hidden4096_every_32nd_block_row(label):
    wl = inputs.hidden4096_block()
    _, ta, tb, M, N, K, an, bn = H4096[label]
    qa, sa, oqa, osa = quantized(wl, an)
    qb, sb, oqb, osb = quantized(wl, bn)
    off = zlib.crc32(label.encode()) % 32
    rows = list(range(off, M // 32, 32))
    note(f"{label}: M={M} N={N} K={K} tA={ta} tB={tb}, block rows {off}::32 ({len(rows)} rows)")
    c, q, s = run_gemm(qa, sa, qb, sb, ta, tb, M, N)
    idx = torch.tensor([32 * I + r for I in rows for r in range(32)], device=DEV)
    gc = host(c.index_select(0, idx))
    gq = host(q.index_select(0, idx))
    gs = host(s.index_select(0, torch.tensor(rows, device=DEV)))
    del c, q, s
    blks = [(I, J) for I in rows for J in range(N // 32)]
    ob = oracle.gemm_f32_blocks(oqa, osa, oqb, osb, blks, ta=ta, tb=tb)      # (nblk, 32, 32)
    ref = ob.reshape(len(rows), N // 32, 32, 32).transpose(0, 2, 1, 3).reshape(32 * len(rows), N)
    exact = check_f32(gc, ref, oqa, osa, oqb, osb, ta, tb, lambda r: rows[r], label)
    rq, rs = oracle.requant(np.ascontiguousarray(ref))
    frac, srel = assert_requant_close(gq, gs, rq, rs, label)
    note(f"  {gc.size} elements: f32 bit-exact {exact:.6f}; i8 code diffs {frac:.2e} "
         f"({int(round(frac * gq.size))} of {gq.size}), scale rel {srel:.1e}")


def exact_expected(A, sA, B, sB, ta, tb):
    """The float64 product of the dequantized operands, on the device, as
    binary32 (checked to be exact in both: the small-code construction)."""
    Ad = torch.from_numpy(oracle.dequantize(A, sA)).to(DEV).double()
    Bd = torch.from_numpy(oracle.dequantize(B, sB)).to(DEV).double()
    exp = torch.matmul(Ad.t().contiguous() if ta else Ad, Bd.t().contiguous() if tb else Bd)
    del Ad, Bd
    assert float(exp.abs().max()) < 2.0 ** 18
    exp32 = exp.float()
    assert torch.equal(exp32.double(), exp), "expected value not exact in binary32"
    return exp32


def small_code_operands(seed, M, N, K, ta, tb):
    """Codes in [-2, 2] and scales in {1/2, 1, 2}, in stored orientation."""
    A = stored(inputs.small_codes(seed, 0, 0, M, K, 2), ta)
    B = stored(inputs.small_codes(seed, 0, 1, K, N, 2), tb)
    sA = stored(inputs.pow2_scales(seed, 0, 2, M // 32, K // 32, -1, 1), ta)
    sB = stored(inputs.pow2_scales(seed, 0, 3, K // 32, N // 32, -1, 1), tb)
    return A, sA, B, sB


def check_exact(c, q, s, exp32, what):
    """Every binary32 output equals the exact product; the INT8 output is
    the oracle's requantization of it (to the INT8 bar)."""
    assert not torch.isnan(c).any(), f"{what}: unwritten (NaN) outputs"
    nbad = int((c != exp32).sum())
    assert nbad == 0, f"{what}: {nbad} binary32 outputs differ from the exact product"
    rq, rs = oracle.requant(host(exp32))
    return assert_requant_close(host(q), host(s), rq, rs, what)


@pytest.mark.parametrize("label", list(H4096))
def test_hidden4096_every_element_exact(label):
    _, ta, tb, M, N, K, _, _ = H4096[label]
    seed = 800 + zlib.crc32(label.encode()) % 1000
    A, sA, B, sB = small_code_operands(seed, M, N, K, ta, tb)
    note(f"{label}: every element, M={M} N={N} K={K} tA={ta} tB={tb}")
    c, q, s = run_gemm(dev(A), dev(sA), dev(B), dev(sB), ta, tb, M, N)
    exp32 = exact_expected(A, sA, B, sB, ta, tb)
    frac, srel = check_exact(c, q, s, exp32, label)
    note(f"  {M * N} elements: f32 exact everywhere; i8 code diffs {frac:.2e}, scale rel {srel:.1e}")


@pytest.mark.parametrize("case", ["main-tile-fwd", "big-tile-wgrad"])
def test_wide_leading_dimension_large_tiles(case):
    """Per-lane load offsets past 32 bits select the kernels' 64-bit address
    path when (ld + 1) * tile edge >= 2^31; with a 256-element tile edge a
    leading dimension of 2^23 + 64 bytes does it.  The forward layout on a
    4096 x 4096 x 256 grid (512 main tiles) with B stored 256 x ld (2.1 GB),
    and the weight-gradient layout on 8192 x 16384 x 2048 (2048 tiles of
    256 x 256, 64 k-blocks) with A stored 2048 x ld (17 GB of HBM); the
    operand sits at the end of each row.  Every element, exact construction."""
    if case == "main-tile-fwd":
        ta, tb, M, N, K = 0, 0, 4096, 4096, 256
    else:
        ta, tb, M, N, K = 1, 0, 8192, 16384, 2048
    A, sA, B, sB = small_code_operands(950 + len(case), M, N, K, ta, tb)
    wide = B if case == "main-tile-fwd" else A
    ld = (1 << 23) + 64
    note(f"wide ld {case}: {M}x{N}x{K} tA={ta} tB={tb}, a {wide.shape[0]} x {ld} operand "
         f"({wide.shape[0] * ld / 2**30:.1f} GiB)")
    big = torch.empty((wide.shape[0], ld), dtype=torch.int8, device=DEV)
    view = big[:, ld - wide.shape[1]:]
    view.copy_(dev(wide))
    qa, qb = (dev(A), view) if case == "main-tile-fwd" else (view, dev(B))
    c, q, s = run_gemm(qa, dev(sA), qb, dev(sB), ta, tb, M, N)
    torch.cuda.synchronize()
    del qa, qb, view, big
    torch.cuda.empty_cache()
    exp32 = exact_expected(A, sA, B, sB, ta, tb)
    frac, srel = check_exact(c, q, s, exp32, case)
    note(f"  {M * N} elements: f32 exact everywhere; i8 code diffs {frac:.2e}, scale rel {srel:.1e}")


GPT2 = [(w, g[0]) for w in ("gpt2_base", "gpt2_medium_mlp") for g in inputs.WORKLOADS[w]().gemms()]


@pytest.mark.parametrize("wname,label", GPT2)
def test_gpt2_workloads_every_element(wname, label):
    wl = inputs.WORKLOADS[wname]()
    _, ta, tb, M, N, K, an, bn = {g[0]: g for g in wl.gemms()}[label]
    qa, sa, oqa, osa = quantized(wl, an)
    qb, sb, oqb, osb = quantized(wl, bn)
    note(f"{wl.name} {label}: M={M} N={N} K={K} tA={ta} tB={tb}, every element")
    c, q, s = run_gemm(qa, sa, qb, sb, ta, tb, M, N)
    gc, gq, gs = host(c), host(q), host(s)
    ref = oracle.gemm_f32(oqa, osa, oqb, osb, ta=ta, tb=tb)
    exact = check_f32(gc, ref, oqa, osa, oqb, osb, ta, tb, lambda r: r, f"{label} f32")
    rq, rs = oracle.requant(ref)
    frac, srel = assert_requant_close(gq, gs, rq, rs, f"{label} i8")
    note(f"  f32 bit-exact {exact:.6f}, i8 code diffs {frac:.2e}, scale rel {srel:.1e}")


@pytest.mark.parametrize("ta,tb", [(0, 1), (1, 0), (1, 1)])
def test_big_tile_ragged_every_element(ta, tb):
    """The 256 x 256 tile (gradient layouts, grids of >= 512 such tiles with
    enough k-blocks) on an 8224 x 4192 output: 33 x 17 tiles with a ragged
    last tile row (one block row of eight) and column (three block columns of
    eight), K = 8192.  Every element with the exact small-code construction,
    and the edge blocks against the oracle with real codes and scales."""
    M, N, K = 8224, 4192, 8192
    seed = 900 + 2 * ta + tb
    A, sA, B, sB = small_code_operands(seed, M, N, K, ta, tb)
    note(f"big tile ragged: {M}x{N}x{K} tA={ta} tB={tb}, every element")
    c, q, s = run_gemm(dev(A), dev(sA), dev(B), dev(sB), ta, tb, M, N)
    exp32 = exact_expected(A, sA, B, sB, ta, tb)
    frac, srel = check_exact(c, q, s, exp32, "big tile ragged (exact)")
    del c, q, s, exp32
    # real codes and scales on the ragged edge blocks
    A = stored(inputs.codes(seed, 1, 0, M, K), ta)
    B = stored(inputs.codes(seed, 1, 1, K, N), tb)
    sA = stored(inputs.scales(seed, 1, 2, M // 32, K // 32), ta)
    sB = stored(inputs.scales(seed, 1, 3, K // 32, N // 32), tb)
    c, q, s = run_gemm(dev(A), dev(sA), dev(B), dev(sB), ta, tb, M, N)
    nbM, nbN = M // 32, N // 32
    blks = sorted({(nbM - 1, J) for J in range(nbN)} | {(I, J) for I in range(0, nbM, 16) for J in range(nbN - 3, nbN)})
    gc, gq, gs = host(c), host(q), host(s)
    oc = oracle.gemm_f32_blocks(A, sA, B, sB, blks, ta=ta, tb=tb)
    np.testing.assert_array_equal(np.stack([gc[32 * I:32 * I + 32, 32 * J:32 * J + 32] for I, J in blks]), oc)
    oq, os_ = oracle.gemm_i8_blocks(A, sA, B, sB, blks, ta=ta, tb=tb)
    frac2, srel2 = assert_requant_close(np.stack([gq[32 * I:32 * I + 32, 32 * J:32 * J + 32] for I, J in blks]),
                                        np.array([gs[I, J] for I, J in blks]), oq, os_, "big tile ragged edges")
    note(f"  exact: f32 exact everywhere, i8 code diffs {frac:.2e}; {len(blks)} edge blocks with real scales: "
         f"f32 bit-exact, i8 code diffs {frac2:.2e}")


# Shapes on both sides of every dispatch switch: the 64 x 128 tile below 512
# main tiles, the 128 x 256 tile from 512, the 256 x 256 tile of the gradient
# layouts from 512 such tiles and 2^17 tile x k-block units, and the
# one-k-block stages for an odd number of k-blocks.
DISPATCH = [
    # (tA, tB, M, N, K, what)
    (0, 0, 4096, 3840, 256, "480 main tiles: 64x128 tile"),
    (0, 0, 4096, 4096, 256, "512 main tiles: 128x256 tile"),
    (0, 1, 4096, 4096, 224, "odd k-block count (7): one-k-block stages"),
    (1, 0, 32, 32, 32, "one block, one k-block"),
    (1, 0, 8192, 4096, 8192, "512 big tiles x 256 k-blocks = 2^17: 256x256 tile"),
    (1, 0, 8192, 4096, 8128, "512 big tiles x 254 k-blocks < 2^17: 128x256 tile"),
    (0, 1, 8192, 3840, 8192, "480 big tiles: 128x256 tile"),
    (1, 1, 8192, 4096, 8192, "both transposed, 256x256 tile"),
]


@pytest.mark.parametrize("ta,tb,M,N,K,what", DISPATCH, ids=[d[5] for d in DISPATCH])
def test_dispatch_boundaries_every_element(ta, tb, M, N, K, what):
    A, sA, B, sB = small_code_operands(1000 + M // 32 + N // 32 + K // 32, M, N, K, ta, tb)
    note(f"dispatch {what}: {M}x{N}x{K} tA={ta} tB={tb}")
    c, q, s = run_gemm(dev(A), dev(sA), dev(B), dev(sB), ta, tb, M, N)
    exp32 = exact_expected(A, sA, B, sB, ta, tb)
    frac, srel = check_exact(c, q, s, exp32, what)
    note(f"  {M * N} elements exact; i8 code diffs {frac:.2e}")


def _sweep_shapes(n=24, seed=2024):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M, N = (int(v) * 32 for v in g.integers(1, 40, size=2))
        K = int(g.integers(1, 70)) * 32
        out.append((int(g.integers(0, 2)), int(g.integers(0, 2)), M, N, K))
    return out


@pytest.mark.parametrize("ta,tb,M,N,K", _sweep_shapes())
def test_seeded_shape_sweep_every_element(ta, tb, M, N, K):
    """Seeded random shapes up to 1248 x 1248 x 2208 in all four layouts
    (small grids, ragged tiles, odd and even k-block counts): every element
    with the exact construction."""
    A, sA, B, sB = small_code_operands(2000 + M + 3 * N + 7 * K + ta + 2 * tb, M, N, K, ta, tb)
    c, q, s = run_gemm(dev(A), dev(sA), dev(B), dev(sB), ta, tb, M, N)
    exp32 = exact_expected(A, sA, B, sB, ta, tb)
    check_exact(c, q, s, exp32, f"{M}x{N}x{K} tA={ta} tB={tb}")
