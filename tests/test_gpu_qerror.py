"""GPU parity: jf_quant_error vs the CPU oracle.

The quantization-error harness behind the per-block vs per-token vs
per-channel comparison (Jetfire summary, "Measured effects").  Bar: group
scales bit-exact; the binary64 error sum within 3 n 2^-53 relative (n
non-negative terms, each rounded once, summed in two different orders: the
recursive-summation bound for each side).  Cases: every granularity on
shapes with ragged groups of four block columns, strided views, the edge
groups (all zero, maxima whose scale underflows to zero, exact half-integer
quotients, negative-only rows), empty matrices, and the 16384 x 16384
memory-bound activations and the GPT2-medium MLP hidden activations in full.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, dev, host, note
from int8_block_quantized_amd import inputs
from int8_block_quantized_amd import jetfire as jf

pytestmark = pytest.mark.gpu

GRANS = ("block", "token", "channel", "tensor")


def sse_tol(n: int) -> float:
    return 3.0 * max(n, 1) * 2.0 ** -53


def check(x_dev: torch.Tensor, x: np.ndarray, gran: str, what: str):
    s, sse = jf.quant_error(x_dev, gran)
    gs, gsse = host(s), float(host(sse)[0])
    os_, osse = oracle.quant_sse(x, gran)
    np.testing.assert_array_equal(gs, os_, err_msg=f"{what} {gran}: scales")
    assert abs(gsse - osse) <= sse_tol(x.size) * osse, f"{what} {gran}: sse {gsse!r} vs {osse!r}"
    return gsse


@pytest.mark.parametrize("gran", GRANS)
@pytest.mark.parametrize("rows,cols", [(96, 160), (64, 96), (32, 32), (128, 512), (256, 1056)])
def test_shapes(gran, rows, cols):
    x = inputs.activation(400 + cols, rows, rows, cols, n_outlier_cols=max(1, cols // 100), factor=50.0)
    sse = check(dev(x), x, gran, f"{rows}x{cols}")
    note(f"quant_error {gran} {rows}x{cols}: mse {sse / x.size:.4e}")


@pytest.mark.parametrize("gran", GRANS)
def test_segments_in_turn_ragged(gran):
    """8192 x 2080: 65 block columns in 9 row segments, so each workgroup takes
    two segments in turn and the last takes one, itself ragged (one block)."""
    rows, cols = 8192, 2080
    x = inputs.activation(420, 0, rows, cols, n_outlier_cols=21, factor=60.0)
    sse = check(dev(x), x, gran, f"{rows}x{cols}")
    note(f"quant_error {gran} {rows}x{cols}: mse {sse / x.size:.4e}")


@pytest.mark.parametrize("gran", GRANS)
def test_strided_view(gran):
    rows, cols = 96, 224
    x = inputs.activation(410, 0, rows, cols, n_outlier_cols=3, factor=80.0)
    big = torch.full((rows, cols + 68), 1e6, dtype=torch.float32, device=DEV)   # pad values would dominate
    big[:, 36:36 + cols] = dev(x)
    check(big[:, 36:36 + cols], x, gran, "strided")


def edge_matrix():
    g = np.random.default_rng(411)
    x = g.normal(size=(96, 192)).astype(np.float32)
    x[0:32, 0:32] = 0.0                                          # all-zero block
    x[0:32, 32:64] = 0.0
    x[3, 40] = np.float32(1e-44)                                 # max/127 underflows: s = 0
    x[7, 50] = -np.float32(3e-45)
    blk = np.arange(-16, 16, dtype=np.float32)[:, None] + np.float32(0.5) * np.ones((1, 32), np.float32)
    x[32:64, 64:96] = blk                                       # half-integer quotients (s = 1 below)
    x[32, 64] = 127.0
    x[64:96, 96:128] = -np.abs(x[64:96, 96:128])                # negative-only block
    x[80, :] = -np.abs(x[80, :])                                 # negative-only row
    x[:, 150] = 0.0                                              # all-zero column
    x[20, :] = 0.0                                               # all-zero row
    return x


@pytest.mark.parametrize("gran", GRANS)
def test_edge_groups(gran):
    x = edge_matrix()
    check(dev(x), x, gran, "edge")


@pytest.mark.parametrize("gran", GRANS)
def test_all_zero(gran):
    x = np.zeros((64, 128), np.float32)
    s, sse = jf.quant_error(dev(x), gran)
    assert np.all(host(s) == 0) and float(host(sse)[0]) == 0.0


@pytest.mark.parametrize("gran", GRANS)
@pytest.mark.parametrize("rows,cols", [(0, 64), (64, 0), (0, 0)])
def test_empty(gran, rows, cols):
    x = torch.zeros((rows, cols), dtype=torch.float32, device=DEV)
    n = jf.scale_count(gran, rows, cols)
    s = torch.full((n,), 5.0, dtype=torch.float32, device=DEV)
    sse = torch.full((1,), 5.0, dtype=torch.float64, device=DEV)
    jf.quant_error(x, gran, s, sse)
    assert np.all(host(s) == 0) and float(host(sse)[0]) == 0.0


def test_repeated_calls_reset_state():
    """The maxima and the sum start from zero on every call (the scale buffer
    doubles as the maxima buffer)."""
    a = inputs.activation(412, 0, 64, 256, n_outlier_cols=2, factor=100.0)
    b = inputs.activation(412, 1, 64, 256, n_outlier_cols=0, factor=1.0)
    s = torch.empty(256, dtype=torch.float32, device=DEV)
    e = torch.empty(1, dtype=torch.float64, device=DEV)
    jf.quant_error(dev(a), "channel", s, e)
    jf.quant_error(dev(b), "channel", s, e)
    os_, osse = oracle.quant_sse(b, "channel")
    np.testing.assert_array_equal(host(s), os_)
    assert abs(float(host(e)[0]) - osse) <= sse_tol(b.size) * osse


def test_hidden_activations_full():
    wl = inputs.gpt2_medium_mlp()
    x = wl.make("H")                                            # 8192 x 4096
    xd = dev(x)
    mse = {g: check(xd, x, g, "mlp hidden") / x.size for g in GRANS}
    note("quant_error mlp hidden 8192x4096 mse: " + ", ".join(f"{g} {v:.4e}" for g, v in mse.items()))
    assert mse["block"] < mse["token"] < mse["tensor"]


def test_memory_bound_workload_full():
    wl = inputs.memory_bound()
    note("quant_error memory-bound: generating")
    x = wl.make("X")                                            # 16384 x 16384
    xd = dev(x)
    for g in GRANS:
        note(f"quant_error memory-bound: {g}")
        check(xd, x, g, "memory-bound")
