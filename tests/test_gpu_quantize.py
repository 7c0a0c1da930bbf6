"""GPU parity: jf_quantize_block / jf_requant_block vs the CPU oracle.

Bar: codes and scales bit-exact (the rule's decisions are binary32 on both
sides).  Cases: the tiny 256x256 workload, a ragged shape, bfloat16 input,
strided (ld > cols) views, edge blocks (zero, underflow, subnormal scale,
exact ties, +-max), several row segments per band with a ragged last one,
a grid split over several launches (2^20 + 64 rows), and the 16384 x 16384
memory-bound workload in full.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, dev, host, note
from int8_block_quantized_amd import inputs
from int8_block_quantized_amd import jetfire as jf

pytestmark = pytest.mark.gpu


def check(x_np, q, s, what):
    oq, os_ = oracle.quantize(x_np)
    np.testing.assert_array_equal(host(s), os_, err_msg=f"{what}: scales")
    np.testing.assert_array_equal(host(q), oq, err_msg=f"{what}: codes")


def test_tiny_workload():
    wl = inputs.tiny_forward()
    for name in ("X", "W", "dY"):
        x = wl.make(name)
        q, s = jf.quantize_block(dev(x))
        check(x, q, s, name)


def test_ragged_and_requant():
    x = inputs.activation(200, 0, 96, 160, n_outlier_cols=3, factor=50.0)
    q, s = jf.quantize_block(dev(x))
    check(x, q, s, "96x160")
    q2, s2 = jf.requant_block(dev(x))
    check(x, q2, s2, "requant 96x160")


def test_bf16_input():
    x = inputs.activation(201, 0, 128, 96, n_outlier_cols=2, factor=50.0)
    xt = torch.from_numpy(x).to(torch.bfloat16)
    bits = xt.view(torch.int16).numpy().view(np.uint16)
    q, s = jf.quantize_block(xt.to(DEV))
    oq, os_ = oracle.quantize(bits)
    np.testing.assert_array_equal(host(s), os_)
    np.testing.assert_array_equal(host(q), oq)


def test_strided_views():
    big = inputs.activation(202, 0, 64, 192, n_outlier_cols=2, factor=50.0)
    xd = dev(big)[:, 32:160]                                  # ld 192 > cols 128
    qbig = torch.full((64, 256), 99, dtype=torch.int8, device=DEV)
    qv = qbig[:, 64:192]                                      # ldq 256
    q, s = jf.quantize_block(xd, q=qv)
    oq, os_ = oracle.quantize(np.ascontiguousarray(big[:, 32:160]))
    np.testing.assert_array_equal(host(s), os_)
    np.testing.assert_array_equal(host(q), oq)
    qb = host(qbig)
    assert np.all(qb[:, :64] == 99) and np.all(qb[:, 192:] == 99), "wrote outside the view"


def test_edge_blocks():
    x = np.zeros((64, 192), np.float32)
    x[3, 32 + 4] = np.float32(1e-45)                          # underflowing scale
    x[0:32, 64:96] = np.float32(1e-37)                        # subnormal scale
    x[1, 64] = np.float32(-3e-37)
    x[0, 96] = 127.0                                          # s = 1: exact ties
    x[1, 96:106] = [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 125.5, 126.5, -126.5]
    g = np.random.default_rng(3)
    x[32:64, 0:32] = g.standard_normal((32, 32)).astype(np.float32)
    x[40, 5] = -x[32:64, 0:32].__abs__().max() * 2            # single negative outlier
    x[32:64, 128:160] = np.float32(-7.25)                     # constant block -> all -127
    x[32:64, 160:192] = np.ldexp(g.integers(-127, 128, (32, 32)).astype(np.float32), -30)
    x[33, 170] = np.ldexp(np.float32(127), -30)
    q, s = jf.quantize_block(dev(x))
    check(x, q, s, "edge blocks")
    qh = host(q)
    assert np.all(qh[32:64, 128:160] == -127)


def test_empty_is_noop():
    x = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    q, s = jf.quantize_block(x)
    assert q.shape == (0, 64) and s.shape == (0, 2)


def test_memory_bound_workload_full():
    wl = inputs.memory_bound()
    note("memory-bound 16384x16384: generating")
    x = wl.make("X")
    note("memory-bound: quantize on GPU")
    q, s = jf.quantize_block(dev(x))
    qh, sh = host(q), host(s)
    note("memory-bound: oracle")
    oq, os_ = oracle.quantize(x)
    np.testing.assert_array_equal(sh, os_)
    np.testing.assert_array_equal(qh, oq)


@pytest.mark.parametrize("rows,cols,dtype", [(320, 800, "f32"), (96, 1056, "bf16"), (64, 2080, "f32")])
def test_several_row_segments_ragged(rows, cols, dtype):
    """Several 1 KiB row segments per 32-row band with a partial last one
    (fp32: 8 blocks per segment, bfloat16: 16)."""
    x = inputs.activation(204, cols, rows, cols, n_outlier_cols=max(1, cols // 100), factor=80.0)
    if dtype == "bf16":
        xt = torch.from_numpy(x).to(torch.bfloat16)
        q, s = jf.quantize_block(xt.to(DEV))
        oq, os_ = oracle.quantize(xt.view(torch.int16).numpy().view(np.uint16))
    else:
        q, s = jf.quantize_block(dev(x))
        oq, os_ = oracle.quantize(x)
    np.testing.assert_array_equal(host(s), os_)
    np.testing.assert_array_equal(host(q), oq)


def test_more_bands_than_one_launch_holds():
    """2^20 + 64 rows: more 32-row bands than one launch's grid dimension
    takes (2^15), so the launcher splits the grid; the band index must carry
    across the launches."""
    rows, cols = (1 << 20) + 64, 64
    note(f"quantize {rows}x{cols}: generating")
    x = inputs.activation(205, 0, rows, cols, n_outlier_cols=1, factor=60.0)
    q, s = jf.quantize_block(dev(x))
    qh, sh = host(q), host(s)
    oq, os_ = oracle.quantize(x)
    np.testing.assert_array_equal(sh, os_)
    np.testing.assert_array_equal(qh, oq)
