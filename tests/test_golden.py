"""The stored fixtures of tests/golden/ (written by tests/golden/make_golden.py
with the CPU oracle): the oracle still reproduces every stored value bit for
bit, and the stored quantization satisfies the rule's invariants checked here
in numpy, independently of the oracle (Jetfire summary, "Approach": one
scale per 32x32 block, s = max|x|/127, codes rne(x/s) in [-127, 127])."""
import numpy as np

import oracle
from golden_io import read


def blocks(a):
    r, c = a.shape
    return a.reshape(r // 32, 32, c // 32, 32).transpose(0, 2, 1, 3)


def test_quantize_fixture():
    d = read("quantize_32x64.txt")
    q, s = oracle.quantize(d["x"])
    np.testing.assert_array_equal(q, d["q"])
    np.testing.assert_array_equal(s, d["s"])
    # invariants, in binary64 numpy: the scale is fl(max|x| / 127) of each
    # block, the block maximum maps to +-127, and |x - s q| <= s/2 up to the
    # rounding of fl(x / s)
    xb, qb = blocks(d["x"].astype(np.float64)), blocks(d["q"].astype(np.float64))
    for i in range(xb.shape[0]):
        for j in range(xb.shape[1]):
            m = np.abs(xb[i, j]).max()
            s_ij = float(d["s"][i, j])
            assert s_ij == float(np.float32(np.float32(m) / np.float32(127)))
            assert np.abs(qb[i, j]).max() == 127
            assert np.all(np.abs(xb[i, j] - s_ij * qb[i, j]) <= s_ij * (0.5 + 2.0 ** -16))


def test_gemm_fixture():
    d = read("gemm_32x32x64.txt")
    np.testing.assert_array_equal(oracle.gemm_f32(d["a"], d["sa"], d["b"], d["sb"]), d["c"])
    qc, sc = oracle.gemm_i8(d["a"], d["sa"], d["b"], d["sb"])
    np.testing.assert_array_equal(qc, d["qc"])
    np.testing.assert_array_equal(sc, d["sc"])
    # the F32 result is the scaled integer product up to the fp32 rounding of
    # the two-term k-block sum (exact rationals bound it)
    a, b = d["a"].astype(np.float64), d["b"].astype(np.float64)
    sa, sb = d["sa"].astype(np.float64), d["sb"].astype(np.float64)
    ref = sum((a[:, 32 * k:32 * k + 32] @ b[32 * k:32 * k + 32]) * float(np.float32(sa[0, k] * sb[k, 0]))
              for k in range(2))
    terms = sum(np.abs(a[:, 32 * k:32 * k + 32] @ b[32 * k:32 * k + 32]) * float(np.float32(sa[0, k] * sb[k, 0]))
                for k in range(2))
    assert np.all(np.abs(d["c"] - ref) <= terms * 2.0 ** -23)


def test_gelu_fixtures():
    d = read("gelu_32x64.txt")
    qo, so = oracle.gelu(d["q"], d["s"])
    np.testing.assert_array_equal(qo, d["qo"])
    np.testing.assert_array_equal(so, d["so"])
    d = read("gelu_bwd_32x64.txt")
    qo, so = oracle.gelu_bwd(d["qdy"], d["sdy"], d["qx"], d["sx"])
    np.testing.assert_array_equal(qo, d["qo"])
    np.testing.assert_array_equal(so, d["so"])


def test_dequant_fixture():
    """The oracle reproduces the stored values, and the stored values hold the
    definition checked independently: y equals the exact product s q wherever
    it is representable (|q| s within binary32 with the product's bits), and
    each bfloat16 pattern is the nearest bfloat16 to y (ties even)."""
    d = read("dequant_32x64.txt")
    for q, s, y, yb in (("q", "s", "y", "ybf16"), ("qx", "sx", "yx", "yxbf16")):
        np.testing.assert_array_equal(oracle.dequantize(d[q], d[s]), d[y])
        np.testing.assert_array_equal(oracle.dequantize_bf16(d[q], d[s]), d[yb])
        exact = np.repeat(np.repeat(d[s].astype(np.float64), 32, 0), 32, 1) * d[q]
        np.testing.assert_array_equal(d[y], exact.astype(np.float32))   # one rounding of the exact product
        up = (d[yb].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.all(np.abs(up - d[y]) <= np.abs(d[y]) * 2.0 ** -8)   # half a bfloat16 ulp (8 bits)


def test_add_layernorm_qerror_fixtures():
    """The oracle reproduces the stored add, LayerNorm and quantization-error
    values bit for bit, and the stored values keep their defining
    invariants: every LayerNorm row has mean ~0 and unit variance before the
    affine map (checked on the stored row statistics against the dequantized
    input), and each granularity's error sum is at most n (s/2)^2 for its
    largest scale."""
    d = read("add_32x64.txt")
    qo, so = oracle.add(d["qa"], d["sa"], d["qb"], d["sb"])
    np.testing.assert_array_equal(qo, d["qo"])
    np.testing.assert_array_equal(so, d["so"])
    d = read("layernorm_32x64.txt")
    qo, so, mean, rstd = oracle.layernorm(d["q"], d["s"], d["gamma"].ravel(), d["beta"].ravel(), 1e-5, stats=True)
    np.testing.assert_array_equal(qo, d["qo"])
    np.testing.assert_array_equal(so, d["so"])
    np.testing.assert_array_equal(mean, d["mean"].ravel())
    np.testing.assert_array_equal(rstd, d["rstd"].ravel())
    x = oracle.dequantize(d["q"], d["s"]).astype(np.float64)
    np.testing.assert_allclose(d["mean"].ravel(), x.mean(axis=1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(d["rstd"].ravel(), 1.0 / np.sqrt(x.var(axis=1) + np.float64(np.float32(1e-5))),
                               rtol=1e-12)
    d = read("qerror_32x64.txt")
    for g in ("block", "token", "channel", "tensor"):
        s, sse = oracle.quant_sse(d["x"], g)
        np.testing.assert_array_equal(s, d[f"s_{g}"].ravel())
        assert sse == float(d[f"sse_{g}"][0, 0])
        assert sse <= d["x"].size * (float(s.max()) / 2) ** 2
