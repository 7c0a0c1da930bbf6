"""GPU: the entry points under HIP graph capture (torch.cuda.graph).

Every entry point enqueues its kernels on the caller's stream, allocates
nothing and never synchronizes, so a sequence of calls can be captured once
and replayed without any host work per kernel.  The captured sequence is one
INT8 linear layer with GELU, forward and backward, plus the other operators:
quantize X, W, dY and a second activation; the block-scaled GEMM with INT8
and binary32 output; GELU; GELU backward; the activation- and weight-gradient
GEMMs; residual add; LayerNorm; dequantization to bfloat16.  Nothing in it
records a memset (the quantization-error entry point, whose atomics need a
cleared buffer, clears it with a kernel but is left out: its binary64 sum is
order-dependent, so replays are not bit-comparable).

The graph is replayed three times.  Before each replay new inputs are copied
into the captured input buffers and unrelated eager work runs on the same
stream; every replay's outputs must equal, bit for bit, the outputs of the
same calls made eagerly on the same inputs (all these kernels are
deterministic).
"""
import numpy as np
import pytest
import torch

from gpu_util import DEV, note
from int8_block_quantized_amd import inputs
from int8_block_quantized_amd import jetfire as jf

pytestmark = pytest.mark.gpu

T, DIN, DOUT = 512, 768, 1024   # tokens, input and output features


def make_inputs(seed):
    g = np.random.default_rng(seed)
    x = inputs.activation(90, seed, T, DIN, 8, 50.0)
    x2 = inputs.activation(91, seed, T, DIN, 8, 50.0)
    w = (g.standard_normal((DIN, DOUT)) * 0.02).astype(np.float32)
    dy = (g.standard_normal((T, DOUT)) * 1e-3).astype(np.float32)
    gamma = (1.0 + 0.1 * g.standard_normal(DIN)).astype(np.float32)
    beta = (0.1 * g.standard_normal(DIN)).astype(np.float32)
    return {n: torch.from_numpy(a).to(DEV) for n, a in
            (("x", x), ("x2", x2), ("w", w), ("dy", dy), ("gamma", gamma), ("beta", beta))}


def layer(t):
    qx, sx = jf.quantize_block(t["x"])
    qx2, sx2 = jf.quantize_block(t["x2"])
    qw, sw = jf.quantize_block(t["w"])
    qd, sd = jf.quantize_block(t["dy"])
    qy, sy = jf.gemm_i8_blockscaled(qx, sx, qw, sw)                       # forward, INT8 out
    cy = jf.gemm_i8_blockscaled(qx, sx, qw, sw, out="f32")                # forward, binary32 out
    qg, sg = jf.gelu_i8(qy, sy)
    qb, sb = jf.gelu_bwd_i8(qd, sd, qy, sy)
    qdx, sdx = jf.gemm_i8_blockscaled(qb, sb, qw, sw, trans_b=True)       # activation gradient
    qdw, sdw = jf.gemm_i8_blockscaled(qx, sx, qb, sb, trans_a=True)       # weight gradient
    qr, sr = jf.add_i8(qx, sx, qx2, sx2)
    qn, sn = jf.layernorm_i8(qr, sr, t["gamma"], t["beta"])
    yb = jf.dequantize_block(qg, sg, dtype=torch.bfloat16)
    return [qx, sx, qw, sw, qd, sd, qy, sy, cy, qg, sg, qb, sb, qdx, sdx, qdw, sdw, qr, sr, qn, sn, yb]


def same(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def test_captured_layer_replays_match_eager():
    static = make_inputs(1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up outside the capture
        layer(static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = layer(static)
    torch.cuda.synchronize()
    other = make_inputs(99)
    for rep in range(3):
        fresh = make_inputs(10 + rep)
        for n in static:
            static[n].copy_(fresh[n])
        layer(other)                       # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        want = layer(fresh)
        torch.cuda.synchronize()
        bad = [i for i, (g_, w_) in enumerate(zip(got, want)) if not same(g_, w_)]
        assert not bad, f"replay {rep}: outputs {bad} differ from the eager calls"
        note(f"graph replay {rep}: {len(got)} outputs bit-identical to eager")
