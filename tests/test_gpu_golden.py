"""GPU parity on the stored fixtures of tests/golden/ (the oracle's outputs on
seeded inputs, written by tests/golden/make_golden.py): quantize and the
block-scaled GEMM (F32 and INT8 output) bit for bit, GELU and GELU backward
to the requantization bar (codes within 1 LSB on at most 0.01% of elements,
scales within 1e-6; the observed differences are printed)."""
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
