"""Writes the fixtures of this folder with the CPU oracle (oracle/) on seeded
synthetic inputs (int8_block_quantized_amd.inputs, workload id 90).  Nothing
else computes a stored value: each expected array is the oracle's output.

The pages print no worked example of the method, so none of these values is
the pages' own; they fix the oracle's results so that a later change of its
arithmetic shows up in tests/test_golden.py, and they give the GPU path a
second, file-based parity check (tests/test_gpu_golden.py).

Run from the repository root:  python3 tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
from golden_io import write  # noqa: E402
from int8_block_quantized_amd import inputs  # noqa: E402

WID = 90
RECIPE = ("inputs: int8_block_quantized_amd.inputs, workload id 90; X = activation(90, 0, 32, 64, "
          "2 columns x100), H = activation(90, 1, 32, 64, 2 columns x100), W = normal(90, W, 0, 64, 32, "
          "std 0.02), dY = normal(90, dY, 0, 32, 64, std 1e-3), gamma = 1 + normal(90, W, 5, 1, 64, std 0.1), "
          "beta = normal(90, W, 6, 1, 64, std 0.1)")


def main():
    x = inputs.activation(WID, 0, 32, 64, 2, 100.0)
    h = inputs.activation(WID, 1, 32, 64, 2, 100.0)
    w = inputs.normal(WID, inputs.TAG_W, 0, 64, 32, 0.02)
    dy = inputs.normal(WID, inputs.TAG_DY, 0, 32, 64, 1e-3)
    qx, sx = oracle.quantize(x)
    qh, sh = oracle.quantize(h)
    qw, sw = oracle.quantize(w)
    qd, sd = oracle.quantize(dy)

    write(os.path.join(HERE, "quantize_32x64.txt"), [
        "Per-block (32x32) quantization of a binary32 matrix: one scale per block,",
        "s = fl(max|x| / 127), q = clamp(rne(fl(x / s)), -127, 127).",
        "Jetfire summary, one-line summary and \"Approach\" (INT8 codes with 32x32 block scales).",
        "Written by tests/golden/make_golden.py with the CPU oracle; " + RECIPE + ".",
    ], [("x", x), ("q", qx), ("s", sx)])

    c = oracle.gemm_f32(qx, sx, qw, sw)
    qc, sc = oracle.gemm_i8(qx, sx, qw, sw)
    write(os.path.join(HERE, "gemm_32x32x64.txt"), [
        "Block-scaled INT8 GEMM C = A B with A = quantize(X) (32 x 64) and B = quantize(W) (64 x 32):",
        "per 32-deep k-block an exact int32 partial P, acc = fma(fl(sA sB), P, acc) in ascending k-block",
        "order (c), then the per-block requantization of acc (qc, sc).",
        "Jetfire summary, \"Approach\" (linear operators on INT8 codes with per-block scales, output",
        "quantized on-chip).",
        "Written by tests/golden/make_golden.py with the CPU oracle; " + RECIPE + ".",
    ], [("a", qx), ("sa", sx), ("b", qw), ("sb", sw), ("c", c), ("qc", qc), ("sc", sc)])

    qg, sg = oracle.gelu(qh, sh)
    write(os.path.join(HERE, "gelu_32x64.txt"), [
        "INT8 GELU with per-block requantization: x = fl(s q), g = x Phi(x) (erf form, binary64,",
        "rounded once), then the per-block rule on g.",
        "Jetfire summary, \"Problem\" and \"Approach\" (non-linear operators also read and write INT8",
        "with block scales).",
        "Written by tests/golden/make_golden.py with the CPU oracle; " + RECIPE + ".",
    ], [("q", qh), ("s", sh), ("qo", qg), ("so", sg)])

    qb, sb = oracle.gelu_bwd(qd, sd, qh, sh)
    write(os.path.join(HERE, "gelu_bwd_32x64.txt"), [
        "INT8 GELU backward: y = fl(fl(s_dy q_dy) GELU'(fl(s_x q_x))), GELU'(x) = Phi(x) + x phi(x) in",
        "binary64 rounded once, then the per-block rule on y.",
        "Jetfire summary, \"Approach\" (every operator of the data flow, the backward pass included, on",
        "INT8 with block scales); the backward of GELU is this library's reading.",
        "Written by tests/golden/make_golden.py with the CPU oracle; " + RECIPE + ".",
    ], [("qdy", qd), ("sdy", sd), ("qx", qh), ("sx", sh), ("qo", qb), ("so", sb)])

    write(os.path.join(HERE, "dequant_32x64.txt"), [
        "Dequantization of per-block INT8 codes (the GELU output above, and quantize(X)): y = fl(s q) in",
        "binary32, and its bfloat16 copy, the nearest bfloat16 of y with ties to even (raw 16-bit patterns).",
        "Jetfire summary, \"Approach\" (INT8 tensors with one scale per 32x32 block).",
        "Written by tests/golden/make_golden.py with the CPU oracle; " + RECIPE + ".",
    ], [("q", qg), ("s", sg), ("y", oracle.dequantize(qg, sg)), ("ybf16", oracle.dequantize_bf16(qg, sg)),
        ("qx", qx), ("sx", sx), ("yx", oracle.dequantize(qx, sx)), ("yxbf16", oracle.dequantize_bf16(qx, sx))])

    qa, sa = oracle.add(qx, sx, qh, sh)
    write(os.path.join(HERE, "add_32x64.txt"), [
        "Residual add of two per-block INT8 tensors (quantize(X) and quantize(H)): z = fl(fl(sa qa) + fl(sb qb)),",
        "then the per-block rule on z.",
        "Jetfire summary, \"Approach\" (every operator of the data flow on INT8 with block scales); the add is",
        "this library's reading.",
        "Written by tests/golden/make_golden.py with the CPU oracle; " + RECIPE + ".",
    ], [("qa", qx), ("sa", sx), ("qb", qh), ("sb", sh), ("qo", qa), ("so", sa)])

    gamma = (1.0 + inputs.normal(WID, inputs.TAG_W, 5, 1, 64, 0.1)).astype(np.float32).ravel()
    beta = inputs.normal(WID, inputs.TAG_W, 6, 1, 64, 0.1).ravel()
    qn, sn, mean, rstd = oracle.layernorm(qx, sx, gamma, beta, 1e-5, stats=True)
    write(os.path.join(HERE, "layernorm_32x64.txt"), [
        "LayerNorm over each row of quantize(X), eps = 1e-5: x = fl(s q); mean and biased variance in binary64",
        "(column order); r = 1/sqrt(v + eps); y = ((x - m) r) gamma + beta in binary64 rounded once to binary32;",
        "then the per-block rule on y (qo, so); the row means and r (binary64).",
        "Jetfire summary, \"Approach\" (INT8 data flow); the normalization is this library's reading.",
        "Written by tests/golden/make_golden.py with the CPU oracle; " + RECIPE + ".",
    ], [("q", qx), ("s", sx), ("gamma", gamma), ("beta", beta), ("qo", qn), ("so", sn), ("mean", mean),
        ("rstd", rstd)])

    arrays = [("x", x)]
    for gname in ("block", "token", "channel", "tensor"):
        sg_, sse = oracle.quant_sse(x, gname)
        arrays += [(f"s_{gname}", sg_), (f"sse_{gname}", np.array([sse], np.float64))]
    write(os.path.join(HERE, "qerror_32x64.txt"), [
        "Quantization error of X under four scale granularities (32x32 block, token = row, channel = column,",
        "tensor): the per-group scale s = fl(max|x| / 127), and sum (x - fl(s q))^2 over all elements, each term",
        "in binary64, added in row order.",
        "Jetfire summary, \"Measured effects\" (per-block against per-token and per-channel quantization error).",
        "Written by tests/golden/make_golden.py with the CPU oracle; " + RECIPE + ".",
    ], arrays)


if __name__ == "__main__":
    main()
