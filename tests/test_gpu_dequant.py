"""GPU parity: jf_dequantize_block (binary32 and bfloat16) vs the CPU oracle.

Bar: bit-exact (every output is one binary32 product, then for bfloat16 one
nearest-even rounding).  Cases: every byte value, scales from subnormal
products to the overflow edge of bfloat16, zero-scale blocks, block-column
counts and row counts that leave a partial tail of the launch grid, strided
input and output views (the padding must stay untouched), the
16384 x 16384 memory-bound workload's GELU output in full, with the data
flow's error against the binary64 GELU of the original fp32 activation, and
the 64-bit index path (2^31 units of work) on sampled block rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, dev, host, note
from int8_block_quantized_amd import inputs
from int8_block_quantized_amd import jetfire as jf

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw patterns of a float32 or bfloat16 device tensor."""
    if t.dtype == torch.bfloat16:
        return host(t.view(torch.int16)).view(np.uint16)
    return host(t).view(np.uint32)


def expected(q, s, dtype):
    if dtype == torch.bfloat16:
        return oracle.dequantize_bf16(q, s)
    return oracle.dequantize(q, s).view(np.uint32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("rows,cols", [(32, 32), (96, 160), (64, 4128), (608, 96)])
def test_random_codes_all_scales(dtype, rows, cols):
    g = np.random.default_rng(rows * 7 + cols)
    q = g.integers(-128, 128, size=(rows, cols)).astype(np.int8)
    s = (10.0 ** g.uniform(-44, 36, size=(rows // 32, cols // 32))).astype(np.float32)
    s.flat[0] = 0.0
    if s.size > 2:
        s.flat[1] = np.float32(3.3895314e38 / 127)     # bfloat16 rounding reaches infinity
        s.flat[2] = np.float32(1e-45)                  # subnormal products
    y = jf.dequantize_block(dev(q), dev(s), dtype=dtype)
    np.testing.assert_array_equal(bits(y), expected(q, s, dtype))
    note(f"dequantize {dtype} {rows}x{cols}: bit-exact")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_strided_views_keep_padding(dtype):
    rows, cols = 96, 224
    g = np.random.default_rng(41)
    q = g.integers(-127, 128, size=(rows, cols)).astype(np.int8)
    s = (10.0 ** g.uniform(-3, 2, size=(rows // 32, cols // 32))).astype(np.float32)
    big_q = torch.zeros((rows, cols + 64), dtype=torch.int8, device=DEV)
    big_q[:, 32:32 + cols] = dev(q)
    big_y = torch.full((rows, cols + 96), 7.0, dtype=dtype, device=DEV)
    jf.dequantize_block(big_q[:, 32:32 + cols], dev(s), dtype=dtype, y=big_y[:, 48:48 + cols])
    got = bits(big_y)
    np.testing.assert_array_equal(got[:, 48:48 + cols], expected(q, s, dtype))
    seven = bits(torch.full((1, 1), 7.0, dtype=dtype, device=DEV))[0, 0]
    assert np.all(got[:, :48] == seven) and np.all(got[:, 48 + cols:] == seven)


def test_empty_is_a_no_op():
    q = torch.empty((0, 64), dtype=torch.int8, device=DEV)
    s = torch.empty((0, 2), dtype=torch.float32, device=DEV)
    assert jf.dequantize_block(q, s, dtype=torch.bfloat16).shape == (0, 64)


def test_memory_bound_gelu_output_bf16_copy():
    """The 16384^2 workload: the oracle's quantized activation and its
    oracle GELU codes go through the GPU dequantization to bfloat16 (every
    element bit-exact against the oracle's copy); that copy then lies within
    the data flow's error bound of the binary64 GELU of the fp32 input:
    input quantization s1 (1/2 + 2e-5) (the code's rounding plus the
    quotient's) times max |GELU'| < 1.13, output code rounding
    s2 (1/2 + 2e-5), and the bfloat16 rounding, half an ulp of 8 significant
    bits: 2^-8 (1 + 2^-7) relative to the rounded value."""
    wl = inputs.memory_bound()
    note("dequantize memory-bound: generating")
    x = wl.make("X")
    oq, os_ = oracle.quantize(x)
    note("dequantize memory-bound: oracle GELU")
    gq, gs = oracle.gelu(oq, os_)
    del oq
    note("dequantize memory-bound: GPU")
    y = jf.dequantize_block(dev(gq), dev(gs), dtype=torch.bfloat16)
    got = bits(y)
    note("dequantize memory-bound: oracle copy")
    np.testing.assert_array_equal(got, oracle.dequantize_bf16(gq, gs))
    del got, gq
    worst = 0.0
    xt = dev(x)
    s1, s2 = dev(os_), dev(gs)
    for r0 in range(0, x.shape[0], 2048):
        xs = xt[r0:r0 + 2048].double()
        ref = 0.5 * xs * torch.special.erfc(-xs / math.sqrt(2.0))
        yb = y[r0:r0 + 2048].double()
        e1 = s1[r0 // 32:(r0 + 2048) // 32].double().repeat_interleave(32, 0).repeat_interleave(32, 1)
        e2 = s2[r0 // 32:(r0 + 2048) // 32].double().repeat_interleave(32, 0).repeat_interleave(32, 1)
        bound = 1.13 * e1 * (0.5 + 2e-5) + e2 * (0.5 + 2e-5) + 2.0 ** -8 * (1 + 2.0 ** -7) * yb.abs() + 1e-30
        worst = max(worst, float(((yb - ref).abs() / bound).max()))
    note(f"dequantize memory-bound: bit-exact; worst error / bound vs binary64 GELU(x) = {worst:.3f}")
    assert worst <= 1.0


@pytest.mark.parametrize("dtype,rows,cols", [(torch.float32, 1 << 17, 1 << 16), (torch.bfloat16, 1 << 18, 1 << 16)],
                         ids=["f32-8Gi-elements", "bf16-16Gi-elements"])
def test_64bit_unit_indices(dtype, rows, cols):
    """At 2^31 units of work (4 codes per unit for binary32 output, 8 for
    bfloat16) the launcher switches to 64-bit unit indices: 8 Gi codes to
    binary32 (40 GB on the device) and 16 Gi codes to bfloat16 (48 GB).
    Codes are drawn on the device; the first, a middle and the last block
    rows are compared with the oracle bit for bit."""
    note(f"dequantize 64-bit indices: {rows} x {cols} to {dtype}")
    g = torch.Generator(device=DEV)
    g.manual_seed(rows + cols)
    q = torch.randint(-127, 128, (rows, cols), dtype=torch.int8, device=DEV, generator=g)
    s = torch.rand((rows // 32, cols // 32), device=DEV, generator=g) * 0.01 + 1e-4
    y = jf.dequantize_block(q, s, dtype=dtype)
    torch.cuda.synchronize()
    for bi in (0, rows // 64, rows // 32 - 1):
        qh = host(q[32 * bi:32 * bi + 32])
        sh = host(s[bi:bi + 1])
        got = bits(y[32 * bi:32 * bi + 32])
        np.testing.assert_array_equal(got, expected(qh, sh, dtype), err_msg=f"block row {bi}")
    del q, s, y
    torch.cuda.empty_cache()
