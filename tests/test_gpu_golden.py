"""GPU parity on the stored fixtures of tests/golden/ (the oracle's outputs on
seeded inputs, written by tests/golden/make_golden.py): quantize, the
block-scaled GEMM (F32 and INT8 output), dequantization, residual add and the
quantization-error scales bit for bit; GELU, GELU backward and LayerNorm to
the requantization bar (codes within 1 LSB on at most 0.01% of elements,
scales within 1e-6; the observed differences are printed); LayerNorm's row
statistics within 1e-13 and the error sums within 3n 2^-53 (summation order)."""
import numpy as np
import pytest

from golden_io import read
from gpu_util import assert_requant_close, dev, host, note
from int8_block_quantized_amd import jetfire as jf

pytestmark = pytest.mark.gpu


def test_quantize_fixture():
    d = read("quantize_32x64.txt")
    q, s = jf.quantize_block(dev(d["x"]))
    np.testing.assert_array_equal(host(q), d["q"])
    np.testing.assert_array_equal(host(s), d["s"])


def test_gemm_fixture():
    d = read("gemm_32x32x64.txt")
    a, sa, b, sb = dev(d["a"]), dev(d["sa"]), dev(d["b"]), dev(d["sb"])
    np.testing.assert_array_equal(host(jf.gemm_i8_blockscaled(a, sa, b, sb, out="f32")), d["c"])
    qc, sc = jf.gemm_i8_blockscaled(a, sa, b, sb, out="i8")
    np.testing.assert_array_equal(host(qc), d["qc"])
    np.testing.assert_array_equal(host(sc), d["sc"])


def test_gelu_fixtures():
    d = read("gelu_32x64.txt")
    qo, so = jf.gelu_i8(dev(d["q"]), dev(d["s"]))
    frac, srel = assert_requant_close(host(qo), host(so), d["qo"], d["so"], "gelu fixture")
    note(f"gelu fixture: code diffs {frac:.2e}, scale rel {srel:.1e}")
    d = read("gelu_bwd_32x64.txt")
    qo, so = jf.gelu_bwd_i8(dev(d["qdy"]), dev(d["sdy"]), dev(d["qx"]), dev(d["sx"]))
    frac, srel = assert_requant_close(host(qo), host(so), d["qo"], d["so"], "gelu_bwd fixture")
    note(f"gelu_bwd fixture: code diffs {frac:.2e}, scale rel {srel:.1e}")


def test_dequant_fixture():
    import torch

    d = read("dequant_32x64.txt")
    for q, s, y, yb in (("q", "s", "y", "ybf16"), ("qx", "sx", "yx", "yxbf16")):
        got = host(jf.dequantize_block(dev(d[q]), dev(d[s])))
        np.testing.assert_array_equal(got.view(np.uint32), d[y].view(np.uint32))
        gb = jf.dequantize_block(dev(d[q]), dev(d[s]), dtype=torch.bfloat16)
        np.testing.assert_array_equal(host(gb.view(torch.int16)).view(np.uint16), d[yb])


def test_add_layernorm_qerror_fixtures():
    d = read("add_32x64.txt")
    qo, so = jf.add_i8(dev(d["qa"]), dev(d["sa"]), dev(d["qb"]), dev(d["sb"]))
    np.testing.assert_array_equal(host(qo), d["qo"])
    np.testing.assert_array_equal(host(so), d["so"])
    d = read("layernorm_32x64.txt")
    qo, so, mean, rstd = jf.layernorm_i8(dev(d["q"]), dev(d["s"]), dev(d["gamma"].ravel()), dev(d["beta"].ravel()),
                                         1e-5, stats=True)
    frac, srel = assert_requant_close(host(qo), host(so), d["qo"], d["so"], "layernorm fixture")
    np.testing.assert_allclose(host(mean), d["mean"].ravel(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(host(rstd), d["rstd"].ravel(), rtol=1e-13)
    note(f"layernorm fixture: code diffs {frac:.2e}, scale rel {srel:.1e}")
    d = read("qerror_32x64.txt")
    n = d["x"].size
    for g in ("block", "token", "channel", "tensor"):
        s, sse = jf.quant_error(dev(d["x"]), g)
        np.testing.assert_array_equal(host(s), d[f"s_{g}"].ravel())
        want = float(d[f"sse_{g}"][0, 0])
        assert abs(float(host(sse)[0]) - want) <= 3 * n * 2.0 ** -53 * want, g
