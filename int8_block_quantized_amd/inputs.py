"""Seeded synthetic inputs for the per-block INT8 data flow.

This module holds only random-number generation: it contains none of the
method's arithmetic (no scale, code, GEMM or GELU computation), so both the
HIP path and the CPU oracle can be fed from it.

Activations follow the pages' description of the data the method is built
for: transformer activations whose trouble is channel-wise outliers (the
Jetfire summary, "Problem" and "Approach").  A "channel" is a column of the
activation matrix (a feature); a fixed set of columns, drawn without
replacement, is scaled by a large factor.

Recipe (all draws are float32 ``standard_normal`` times the stated standard
deviation):
  * generator  ``numpy.random.default_rng([workload_id, tensor_tag, index])``;
  * tags: activation X = 0, weight W = 1, output gradient dY = 2,
    outlier-column choice = 3;
  * ``N(0, sigma)`` means standard deviation sigma.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TAG_X, TAG_W, TAG_DY, TAG_OUTLIER = 0, 1, 2, 3


def rng(workload_id: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(workload_id), int(tag), int(index)])


def normal(workload_id: int, tag: int, index: int, rows: int, cols: int, std: float) -> np.ndarray:
    """rows x cols float32 draws with standard deviation ``std``."""
    g = rng(workload_id, tag, index)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def outlier_columns(workload_id: int, index: int, cols: int, n_cols: int) -> np.ndarray:
    g = rng(workload_id, TAG_OUTLIER, index)
    return np.sort(g.choice(cols, size=n_cols, replace=False))


def activation(workload_id: int, index: int, rows: int, cols: int,
               n_outlier_cols: int, factor: float) -> np.ndarray:
    """N(0, 1) activations with ``n_outlier_cols`` columns scaled by ``factor``."""
    x = normal(workload_id, TAG_X, index, rows, cols, 1.0)
    if n_outlier_cols:
        x[:, outlier_columns(workload_id, index, cols, n_outlier_cols)] *= np.float32(factor)
    return x


def codes(workload_id: int, tag: int, index: int, rows: int, cols: int) -> np.ndarray:
    """Uniform int8 codes in [-127, 127] (random operands for GEMM tests)."""
    return rng(workload_id, tag, index).integers(-127, 128, size=(rows, cols)).astype(np.int8)


def scales(workload_id: int, tag: int, index: int, rows: int, cols: int) -> np.ndarray:
    """Positive float32 values spread over three decades (random scale grids)."""
    g = rng(workload_id, tag, index)
    mant = g.random((rows, cols)) * 1.5 + 0.5
    return (mant * 10.0 ** g.integers(-4, -1, size=(rows, cols))).astype(np.float32)


def small_codes(workload_id: int, tag: int, index: int, rows: int, cols: int, qmax: int) -> np.ndarray:
    """Uniform int8 codes in [-qmax, qmax]."""
    return rng(workload_id, tag, index).integers(-qmax, qmax + 1, size=(rows, cols)).astype(np.int8)


def pow2_scales(workload_id: int, tag: int, index: int, rows: int, cols: int, emin: int, emax: int) -> np.ndarray:
    """float32 powers of two 2^e with e uniform in [emin, emax]."""
    e = rng(workload_id, tag, index).integers(emin, emax + 1, size=(rows, cols))
    return np.ldexp(np.ones((rows, cols), np.float32), e).astype(np.float32)


def n_outliers(fraction: float, cols: int) -> int:
    return int(round(fraction * cols))


# ---------------------------------------------------------------------------
# Workloads.  Each GEMM is (name, transA, transB, M, N, K, a_tensor, b_tensor)
# with W stored as the logical K x N (in_features x out_features) matrix:
#   forward  Y  = X  . W    -> (tA, tB) = (0, 0)
#   dgrad    dX = dY . W^T  -> (0, 1)
#   wgrad    dW = X^T . dY  -> (1, 0)
# ---------------------------------------------------------------------------


@dataclass
class Linear:
    name: str
    m: int          # tokens
    k: int          # in features
    n: int          # out features
    x: str          # name of the input activation tensor (m x k)
    w: str          # name of the weight tensor (k x n)
    dy: str         # name of the output gradient tensor (m x n)

    def gemms(self):
        """The three GEMMs of one linear layer as (label, tA, tB, M, N, K, a, b)."""
        return [
            (f"{self.name}.fwd", 0, 0, self.m, self.n, self.k, self.x, self.w),
            (f"{self.name}.dgrad", 0, 1, self.m, self.k, self.n, self.dy, self.w),
            (f"{self.name}.wgrad", 1, 0, self.k, self.n, self.m, self.x, self.dy),
        ]


@dataclass
class Workload:
    wid: int
    name: str
    tensors: dict = field(default_factory=dict)   # name -> (kind, rows, cols, params)
    linears: list = field(default_factory=list)

    def make(self, name: str) -> np.ndarray:
        kind, rows, cols, p = self.tensors[name]
        idx = list(self.tensors).index(name)
        if kind == "act":
            return activation(self.wid, idx, rows, cols, p["n_out"], p["factor"])
        if kind == "w":
            return normal(self.wid, TAG_W, idx, rows, cols, p["std"])
        if kind == "dy":
            return normal(self.wid, TAG_DY, idx, rows, cols, p["std"])
        raise KeyError(kind)

    def gemms(self):
        out = []
        for lin in self.linears:
            out.extend(lin.gemms())
        return out

    def gemm_ops(self) -> int:
        return sum(2 * M * N * K for (_, _, _, M, N, K, _, _) in self.gemms())


def tiny_forward() -> Workload:
    """256x256 activations (N(0,1), 4 columns x50) times a 256x256 N(0,0.02)
    weight: one forward GEMM."""
    w = Workload(0, "tiny forward 256x256x256")
    w.tensors = {
        "X": ("act", 256, 256, {"n_out": 4, "factor": 50.0}),
        "W": ("w", 256, 256, {"std": 0.02}),
        "dY": ("dy", 256, 256, {"std": 1e-3}),
    }
    w.linears = [Linear("fc", 256, 256, 256, "X", "W", "dY")]
    return w


def gpt2_base_linear() -> Workload:
    """GPT2-base-like linear: tokens M=4096 (4x1024), 768 -> 3072."""
    w = Workload(1, "GPT2-base linear 4096 tokens 768->3072")
    w.tensors = {
        "X": ("act", 4096, 768, {"n_out": n_outliers(0.01, 768), "factor": 50.0}),
        "W": ("w", 768, 3072, {"std": 0.02}),
        "dY": ("dy", 4096, 3072, {"std": 1e-3}),
    }
    w.linears = [Linear("fc", 4096, 768, 3072, "X", "W", "dY")]
    return w


def gpt2_medium_mlp() -> Workload:
    """GPT2-medium-like MLP: 8192 tokens, FC1 1024->4096, GELU, FC2 4096->1024.
    FC2's input is the INT8 GELU output of FC1 (``H`` is only its shape)."""
    w = Workload(2, "GPT2-medium MLP 8192 tokens 1024->4096->1024")
    w.tensors = {
        "X": ("act", 8192, 1024, {"n_out": n_outliers(0.01, 1024), "factor": 50.0}),
        "W1": ("w", 1024, 4096, {"std": 0.02}),
        "W2": ("w", 4096, 1024, {"std": 0.02}),
        "dY2": ("dy", 8192, 1024, {"std": 1e-3}),
        "dY1": ("dy", 8192, 4096, {"std": 1e-3}),
        "H": ("act", 8192, 4096, {"n_out": n_outliers(0.01, 4096), "factor": 50.0}),
    }
    w.linears = [Linear("fc1", 8192, 1024, 4096, "X", "W1", "dY1"),
                 Linear("fc2", 8192, 4096, 1024, "H", "W2", "dY2")]
    return w


def hidden4096_block() -> Workload:
    """Hidden-4096 transformer-block linears, 8192 tokens (8x1024):
    QKV 4096->12288, out-proj 4096->4096, FC1 4096->16384, FC2 16384->4096.
    Activations N(0,1) with 0.5% of columns x100; weights N(0,0.02); output
    gradients N(0,1e-3)."""
    T = 8192
    w = Workload(3, "hidden-4096 block linears 8192 tokens")
    act = lambda c: {"n_out": n_outliers(0.005, c), "factor": 100.0}
    w.tensors = {
        "X": ("act", T, 4096, act(4096)),          # QKV and FC1 input
        "A": ("act", T, 4096, act(4096)),          # attention output (out-proj input)
        "H": ("act", T, 16384, act(16384)),        # FC2 input
        "Wqkv": ("w", 4096, 12288, {"std": 0.02}),
        "Wo": ("w", 4096, 4096, {"std": 0.02}),
        "W1": ("w", 4096, 16384, {"std": 0.02}),
        "W2": ("w", 16384, 4096, {"std": 0.02}),
        "dQKV": ("dy", T, 12288, {"std": 1e-3}),
        "dO": ("dy", T, 4096, {"std": 1e-3}),
        "dH": ("dy", T, 16384, {"std": 1e-3}),
        "dY": ("dy", T, 4096, {"std": 1e-3}),
    }
    w.linears = [Linear("qkv", T, 4096, 12288, "X", "Wqkv", "dQKV"),
                 Linear("out", T, 4096, 4096, "A", "Wo", "dO"),
                 Linear("fc1", T, 4096, 16384, "X", "W1", "dH"),
                 Linear("fc2", T, 16384, 4096, "H", "W2", "dY")]
    return w


def memory_bound() -> Workload:
    """16384 x 16384 N(0,1) activations with 1% of columns x100: quantize,
    then INT8 GELU with per-block requantization."""
    w = Workload(4, "memory-bound 16384x16384")
    w.tensors = {"X": ("act", 16384, 16384, {"n_out": n_outliers(0.01, 16384), "factor": 100.0})}
    return w


WORKLOADS = {
    "tiny": tiny_forward,
    "gpt2_base": gpt2_base_linear,
    "gpt2_medium_mlp": gpt2_medium_mlp,
    "hidden4096": hidden4096_block,
    "memory_bound": memory_bound,
}
