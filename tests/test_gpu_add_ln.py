"""GPU parity: jf_add_i8 and jf_layernorm_i8 vs the CPU oracle.

Residual add: every step is one binary32 rounding of the same operations on
both sides, so codes and scales must be bit-exact.  LayerNorm: the binary64
row sums are added in a different order on the GPU, so y may differ in its
last binary32 bit where the binary64 value sits on a rounding boundary; bar:
codes within 1 LSB on at most 0.01% of elements, scales within 1e-6
relative, row statistics within 1e-13 (rstd relative; the mean relative to
the row's mean magnitude, since it may cancel to ~0).  Observed differences
are printed.  Cases: ragged groups of four block columns, strided views,
edge blocks (zero scales, cancellation, constant rows, the byte -128),
rows held in registers (up to 4096 columns) and rows re-read per pass
(wider), and the hidden-4096 and GPT2-medium activations in full.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, assert_requant_close, dev, host, note
from int8_block_quantized_amd import inputs
from int8_block_quantized_amd import jetfire as jf

pytestmark = pytest.mark.gpu


def codes_of(seed, rows, cols, n_out=3, factor=50.0):
    x = inputs.activation(seed, 0, rows, cols, n_outlier_cols=n_out, factor=factor)
    return oracle.quantize(x)


# ---------------------------------------------------------------- add


@pytest.mark.parametrize("rows,cols", [(32, 32), (64, 96), (96, 160), (128, 544), (256, 1024)])
def test_add_shapes(rows, cols):
    qa, sa = codes_of(500 + cols, rows, cols)
    qb, sb = codes_of(600 + cols, rows, cols, n_out=1, factor=5.0)
    qo, so = jf.add_i8(dev(qa), dev(sa), dev(qb), dev(sb))
    eq, es = oracle.add(qa, sa, qb, sb)
    np.testing.assert_array_equal(host(so), es)
    np.testing.assert_array_equal(host(qo), eq)


def test_add_edge_blocks():
    g = np.random.default_rng(501)
    qa = g.integers(-128, 128, size=(64, 160)).astype(np.int8)          # -128 included
    qb = g.integers(-128, 128, size=(64, 160)).astype(np.int8)
    sa = (10.0 ** g.uniform(-6, 3, size=(2, 5))).astype(np.float32)
    sb = (10.0 ** g.uniform(-6, 3, size=(2, 5))).astype(np.float32)
    sa[0, 0] = sb[0, 0] = 0.0                                          # both zero
    sa[0, 1] = 0.0                                                     # one zero
    qb[0:32, 64:96] = -qa[0:32, 64:96]                                 # exact cancellation
    sb[0, 2] = sa[0, 2]
    qa[32:64, 0:32] = qb[32:64, 0:32] = 0                              # zero codes
    qo, so = jf.add_i8(dev(qa), dev(sa), dev(qb), dev(sb))
    eq, es = oracle.add(qa, sa, qb, sb)
    np.testing.assert_array_equal(host(so), es)
    np.testing.assert_array_equal(host(qo), eq)


def test_add_strided_views():
    rows, cols = 96, 224
    qa, sa = codes_of(502, rows, cols)
    qb, sb = codes_of(503, rows, cols)
    big_a = torch.zeros((rows, cols + 48), dtype=torch.int8, device=DEV)
    big_a[:, 16:16 + cols] = dev(qa)
    big_b = torch.zeros((rows, cols + 96), dtype=torch.int8, device=DEV)
    big_b[:, 64:64 + cols] = dev(qb)
    big_o = torch.full((rows, cols + 64), 7, dtype=torch.int8, device=DEV)
    so = torch.empty((rows // 32, cols // 32), dtype=torch.float32, device=DEV)
    jf.add_i8(big_a[:, 16:16 + cols], dev(sa), big_b[:, 64:64 + cols], dev(sb), big_o[:, 32:32 + cols], so)
    got = host(big_o)
    eq, es = oracle.add(qa, sa, qb, sb)
    np.testing.assert_array_equal(got[:, 32:32 + cols], eq)
    np.testing.assert_array_equal(host(so), es)
    assert np.all(got[:, :32] == 7) and np.all(got[:, 32 + cols:] == 7)


def test_add_residual_stream_full():
    """The hidden-4096 workload's residual add: X (8192 x 4096) + A."""
    wl = inputs.hidden4096_block()
    qa, sa = oracle.quantize(wl.make("X"))
    qb, sb = oracle.quantize(wl.make("A"))
    qo, so = jf.add_i8(dev(qa), dev(sa), dev(qb), dev(sb))
    eq, es = oracle.add(qa, sa, qb, sb)
    np.testing.assert_array_equal(host(so), es)
    np.testing.assert_array_equal(host(qo), eq)


# ---------------------------------------------------------- LayerNorm


def affine(seed, cols):
    g = np.random.default_rng(seed)
    return (g.normal(1.0, 0.3, size=cols).astype(np.float32), g.normal(0.0, 0.2, size=cols).astype(np.float32))


def check_ln(q, s, gamma, beta, eps, what, q_dev=None, out=None):
    qd = dev(q) if q_dev is None else q_dev
    if out is None:
        qo, so, mean, rstd = jf.layernorm_i8(qd, dev(s), dev(gamma), dev(beta), eps, stats=True)
        got_q = host(qo)
    else:
        big_o, sl = out
        so = torch.empty((q.shape[0] // 32, q.shape[1] // 32), dtype=torch.float32, device=DEV)
        _, _, mean, rstd = jf.layernorm_i8(qd, dev(s), dev(gamma), dev(beta), eps, qo=big_o[sl], so=so, stats=True)
        got_q = host(big_o)[sl]
    eq, es, em, er = oracle.layernorm(q, s, gamma, beta, eps, stats=True)
    frac, srel = assert_requant_close(got_q, host(so), eq, es, what)
    # the mean against the row's mean magnitude (it may cancel to ~0); rstd relative
    mag = np.abs(oracle.dequantize(q, s).astype(np.float64)).mean(axis=1)
    err_m = np.abs(host(mean) - em) / np.maximum(np.abs(em) + mag, 1e-300)
    err_r = np.abs(host(rstd) - er) / er
    assert err_m.max() <= 1e-13, f"{what}: mean err {err_m.max():.2e}"
    assert err_r.max() <= 1e-13, f"{what}: rstd rel err {err_r.max():.2e}"
    note(f"layernorm {what}: code diffs {frac:.2e}, scale rel {srel:.1e}")


@pytest.mark.parametrize("rows,cols", [(32, 32), (64, 96), (96, 160), (64, 1024), (32, 2048), (32, 4096),
                                       (64, 4224), (32, 8192)])
def test_layernorm_shapes(rows, cols):
    q, s = codes_of(700 + cols, rows, cols, n_out=max(1, cols // 200), factor=100.0)
    gamma, beta = affine(701 + cols, cols)
    check_ln(q, s, gamma, beta, 1e-5, f"{rows}x{cols}")


def test_layernorm_edge_rows():
    rows, cols = 96, 352                                                # 11 block columns: ragged groups
    q, s = codes_of(702, rows, cols)
    q[0:32, :] = 9                                                      # constant rows (variance 0) ...
    s[0, :] = 0.5                                                       # ... over equal scales
    s[1, 3] = 0.0                                                       # a zero-scale block
    q[64:96, 32:64] = -128                                              # the byte -128
    gamma, beta = affine(703, cols)
    gamma[5] = 0.0
    beta[:32] = 0.0                                                     # a block column with gamma*0 + 0
    gamma[:32] = 0.0
    check_ln(q, s, gamma, beta, 1e-5, "edge rows")


def test_layernorm_eps_zero():
    q, s = codes_of(704, 64, 256)
    gamma, beta = affine(705, 256)
    check_ln(q, s, gamma, beta, 0.0, "eps 0")


def test_layernorm_strided_views():
    rows, cols = 64, 1056
    q, s = codes_of(706, rows, cols)
    gamma, beta = affine(707, cols)
    big = torch.zeros((rows, cols + 32), dtype=torch.int8, device=DEV)
    big[:, 16:16 + cols] = dev(q)
    big_o = torch.full((rows, cols + 80), 7, dtype=torch.int8, device=DEV)
    check_ln(q, s, gamma, beta, 1e-5, "strided", q_dev=big[:, 16:16 + cols],
             out=(big_o, (slice(None), slice(48, 48 + cols))))
    got = host(big_o)
    assert np.all(got[:, :48] == 7) and np.all(got[:, 48 + cols:] == 7)


def test_layernorm_without_stats():
    q, s = codes_of(708, 64, 512)
    gamma, beta = affine(709, 512)
    qo, so = jf.layernorm_i8(dev(q), dev(s), dev(gamma), dev(beta))
    eq, es = oracle.layernorm(q, s, gamma, beta)
    assert_requant_close(host(qo), host(so), eq, es, "no stats")


@pytest.mark.parametrize("which", ["hidden4096", "gpt2_medium"])
def test_layernorm_workload_full(which):
    wl = inputs.hidden4096_block() if which == "hidden4096" else inputs.gpt2_medium_mlp()
    x = wl.make("X")                                                    # 8192 x 4096 / 8192 x 1024
    q, s = oracle.quantize(x)
    gamma, beta = affine(710, x.shape[1])
    check_ln(q, s, gamma, beta, 1e-5, f"{which} {x.shape[0]}x{x.shape[1]}")
