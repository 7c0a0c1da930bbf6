"""The seeded input generators against the workload recipe (CPU).

The synthetic workloads stand in for the pages' data (transformer
activations with channel-wise outliers, small weights, small gradients); this
pins the generators to the stated recipe so that a change of shapes, outlier
fractions or scales cannot go unnoticed: shapes and GEMM lists of every
workload, determinism under the seed, the outlier columns (count, factor,
nothing else scaled) and the standard deviations.
"""
import numpy as np
import pytest

from int8_block_quantized_amd import inputs

EXPECTED_GEMMS = {
    "tiny": [("fc.fwd", 0, 0, 256, 256, 256), ("fc.dgrad", 0, 1, 256, 256, 256), ("fc.wgrad", 1, 0, 256, 256, 256)],
    "gpt2_base": [("fc.fwd", 0, 0, 4096, 3072, 768), ("fc.dgrad", 0, 1, 4096, 768, 3072),
                  ("fc.wgrad", 1, 0, 768, 3072, 4096)],
    "gpt2_medium_mlp": [("fc1.fwd", 0, 0, 8192, 4096, 1024), ("fc1.dgrad", 0, 1, 8192, 1024, 4096),
                        ("fc1.wgrad", 1, 0, 1024, 4096, 8192), ("fc2.fwd", 0, 0, 8192, 1024, 4096),
                        ("fc2.dgrad", 0, 1, 8192, 4096, 1024), ("fc2.wgrad", 1, 0, 4096, 1024, 8192)],
    "hidden4096": [("qkv.fwd", 0, 0, 8192, 12288, 4096), ("qkv.dgrad", 0, 1, 8192, 4096, 12288),
                   ("qkv.wgrad", 1, 0, 4096, 12288, 8192), ("out.fwd", 0, 0, 8192, 4096, 4096),
                   ("out.dgrad", 0, 1, 8192, 4096, 4096), ("out.wgrad", 1, 0, 4096, 4096, 8192),
                   ("fc1.fwd", 0, 0, 8192, 16384, 4096), ("fc1.dgrad", 0, 1, 8192, 4096, 16384),
                   ("fc1.wgrad", 1, 0, 4096, 16384, 8192), ("fc2.fwd", 0, 0, 8192, 4096, 16384),
                   ("fc2.dgrad", 0, 1, 8192, 16384, 4096), ("fc2.wgrad", 1, 0, 16384, 4096, 8192)],
}


@pytest.mark.parametrize("name", list(EXPECTED_GEMMS))
def test_gemm_lists(name):
    wl = inputs.WORKLOADS[name]()
    assert [g[:6] for g in wl.gemms()] == EXPECTED_GEMMS[name]
    for (_, ta, tb, M, N, K, an, bn) in wl.gemms():
        ar, ac = wl.tensors[an][1:3]
        br, bc = wl.tensors[bn][1:3]
        assert (ar, ac) == ((K, M) if ta else (M, K))
        assert (br, bc) == ((N, K) if tb else (K, N))


def test_hidden4096_step_ops():
    assert inputs.hidden4096_block().gemm_ops() == 9895604649984


def test_deterministic_and_distinct():
    a = inputs.activation(3, 0, 256, 512, 3, 100.0)
    np.testing.assert_array_equal(a, inputs.activation(3, 0, 256, 512, 3, 100.0))
    assert not np.array_equal(a, inputs.activation(3, 1, 256, 512, 3, 100.0))
    assert not np.array_equal(a, inputs.activation(4, 0, 256, 512, 3, 100.0))


@pytest.mark.parametrize("name,tensor,frac,factor", [("hidden4096", "X", 0.005, 100.0),
                                                     ("gpt2_base", "X", 0.01, 50.0),
                                                     ("gpt2_medium_mlp", "X", 0.01, 50.0)])
def test_outlier_columns(name, tensor, frac, factor):
    """The stated fraction of columns is scaled by the stated factor and
    nothing else is: with the same draws unscaled, the ratio is exactly the
    factor on those columns and 1 elsewhere."""
    wl = inputs.WORKLOADS[name]()
    kind, rows, cols, p = wl.tensors[tensor]
    rows = min(rows, 512)                                  # the column choice does not depend on rows
    idx = list(wl.tensors).index(tensor)
    x = inputs.activation(wl.wid, idx, rows, cols, p["n_out"], p["factor"])
    base = inputs.normal(wl.wid, inputs.TAG_X, idx, rows, cols, 1.0)
    cols_out = inputs.outlier_columns(wl.wid, idx, cols, p["n_out"])
    assert p["factor"] == factor and len(cols_out) == p["n_out"] == inputs.n_outliers(frac, cols)
    assert abs(len(cols_out) - frac * cols) <= 1
    scaled = np.zeros(cols, bool)
    scaled[cols_out] = True
    np.testing.assert_array_equal(x[:, ~scaled], base[:, ~scaled])
    np.testing.assert_array_equal(x[:, scaled], base[:, scaled] * np.float32(factor))


@pytest.mark.parametrize("tensor,std", [("Wqkv", 0.02), ("dQKV", 1e-3)])
def test_standard_deviations(tensor, std):
    wl = inputs.hidden4096_block()
    kind, rows, cols, p = wl.tensors[tensor]
    idx = list(wl.tensors).index(tensor)
    tag = inputs.TAG_W if kind == "w" else inputs.TAG_DY
    x = inputs.normal(wl.wid, tag, idx, 256, cols, p["std"])
    assert p["std"] == std
    assert abs(float(x.std()) / std - 1.0) < 0.01 and abs(float(x.mean())) < 0.01 * std
