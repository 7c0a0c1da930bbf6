"""CPU oracle for the per-block (32x32) INT8 data flow.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library never loads it, and it shares no code with the HIP path.

This module is the ctypes binding of ``oracle/jfo.c`` (the plain C
reference) plus the numpy marshalling around it.  Every function takes and
returns contiguous numpy arrays; shapes are multiples of 32.

Method source: "Jetfire: Efficient and Accurate Transformer Pretraining with
INT8 Data Flow and Per-Block Quantization" (scime.ai summary of arXiv
2403.12422), one-line summary and "Approach" (per-block 32x32 scales, INT8 in
and out of every linear and non-linear operator, INT8 weight gradient).
The formulas are readings of that text; ``jfo.c`` states each one.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against exact rational arithmetic, closed forms, mpmath and numpy integer
matmul; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "jfo.c")
LIB_PATH = os.path.join(_HERE, "libjfo.so")

# -O2 only: no -march=native (the library may run on another host CPU), no
# fast-math, and no FMA contraction so every rounding is the one written.
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=gnu11"]


def build(verbose: bool = False) -> str:
    """Compile jfo.c into libjfo.so next to it (always recompiles)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        i64, ptr = ctypes.c_int64, ctypes.c_void_p
        lib.jfo_quantize_f32.argtypes = [ptr, i64, i64, ptr, ptr]
        lib.jfo_quantize_bf16.argtypes = [ptr, i64, i64, ptr, ptr]
        lib.jfo_requant.argtypes = [ptr, i64, i64, ptr, ptr]
        lib.jfo_dequantize.argtypes = [ptr, ptr, i64, i64, ptr]
        lib.jfo_dequantize_bf16.argtypes = [ptr, ptr, i64, i64, ptr]
        lib.jfo_bf16_round.argtypes = [ptr, i64, ptr]
        lib.jfo_gemm_f32.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, ptr, ptr, ptr, ptr, ptr]
        lib.jfo_gemm_f32_blocks.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                            ptr, ptr, ptr, ptr, ptr, i64, ptr]
        lib.jfo_gemm_partial.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                         ptr, ptr, i64, i64, i64, ptr]
        lib.jfo_gemm_i8.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                    ptr, ptr, ptr, ptr, ptr, ptr]
        lib.jfo_gemm_i8_blocks.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                           ptr, ptr, ptr, ptr, ptr, i64, ptr, ptr]
        lib.jfo_gelu.argtypes = [ptr, ptr, i64, i64, ptr, ptr]
        lib.jfo_gelu_value.argtypes = [ctypes.c_float]
        lib.jfo_gelu_value.restype = ctypes.c_float
        lib.jfo_gelu_bwd.argtypes = [ptr, ptr, ptr, ptr, i64, i64, ptr, ptr]
        lib.jfo_gelu_grad_value.argtypes = [ctypes.c_float]
        lib.jfo_gelu_grad_value.restype = ctypes.c_float
        lib.jfo_quant_groups.argtypes = [ctypes.c_int, i64, i64]
        lib.jfo_quant_groups.restype = i64
        lib.jfo_quant_sse.argtypes = [ptr, i64, i64, ctypes.c_int, ptr, ptr]
        lib.jfo_add.argtypes = [ptr, ptr, ptr, ptr, i64, i64, ptr, ptr]
        lib.jfo_layernorm.argtypes = [ptr, ptr, i64, i64, ptr, ptr, ctypes.c_float, ptr, ptr, ptr, ptr]
        lib.jfo_set_threads.argtypes = [ctypes.c_int]
        lib.jfo_get_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _chk(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad arguments (rc={rc})")


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def set_threads(n: int) -> None:
    _load().jfo_set_threads(int(n))


def get_threads() -> int:
    return int(_load().jfo_get_threads())


def quantize(x: np.ndarray):
    """Per-block quantization of a 2-D binary32 (or bfloat16 bit-pattern
    uint16) array.  Returns (codes int8 [R,C], scales float32 [R/32,C/32])."""
    x = np.ascontiguousarray(x)
    R, C = x.shape
    q = np.empty((R, C), np.int8)
    s = np.empty((R // 32, C // 32), np.float32)
    if x.dtype == np.float32:
        _chk(_load().jfo_quantize_f32(_p(x), R, C, _p(q), _p(s)), "quantize")
    elif x.dtype == np.uint16:
        _chk(_load().jfo_quantize_bf16(_p(x), R, C, _p(q), _p(s)), "quantize_bf16")
    else:
        raise TypeError("quantize takes float32 or bfloat16 bits (uint16)")
    return q, s


def requant(x: np.ndarray):
    """Per-block requantization of a binary32 array (same rule as quantize)."""
    x = _c(x, np.float32)
    R, C = x.shape
    q = np.empty((R, C), np.int8)
    s = np.empty((R // 32, C // 32), np.float32)
    _chk(_load().jfo_requant(_p(x), R, C, _p(q), _p(s)), "requant")
    return q, s


def dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    R, C = q.shape
    out = np.empty((R, C), np.float32)
    _chk(_load().jfo_dequantize(_p(q), _p(s), R, C, _p(out)), "dequantize")
    return out


def dequantize_bf16(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """bfloat16 copy of fl(s * q): nearest bfloat16, ties to even, as the raw
    16-bit patterns (uint16)."""
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    R, C = q.shape
    out = np.empty((R, C), np.uint16)
    _chk(_load().jfo_dequantize_bf16(_p(q), _p(s), R, C, _p(out)), "dequantize_bf16")
    return out


def bf16_round(f: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 (ties to even) of each finite binary32 value, as uint16 patterns."""
    f = np.ascontiguousarray(f, dtype=np.float32).ravel()
    out = np.empty(f.shape, np.uint16)
    _chk(_load().jfo_bf16_round(_p(f), f.size, _p(out)), "bf16_round")
    return out


def _gemm_dims(ta, tb, A, B):
    M, K = (A.shape[1], A.shape[0]) if ta else A.shape
    K2, N = (B.shape[1], B.shape[0]) if tb else B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    return M, N, K


def gemm_f32(A, sA, B, sB, ta=0, tb=0) -> np.ndarray:
    """C = op(A) op(B) with binary32 output (block-ordered fused sum)."""
    A, B = _c(A, np.int8), _c(B, np.int8)
    sA, sB = _c(sA, np.float32), _c(sB, np.float32)
    M, N, K = _gemm_dims(ta, tb, A, B)
    C = np.empty((M, N), np.float32)
    _chk(_load().jfo_gemm_f32(int(ta), int(tb), M, N, K, _p(A), _p(sA), _p(B), _p(sB), _p(C)), "gemm_f32")
    return C


def gemm_f32_blocks(A, sA, B, sB, blocks, ta=0, tb=0) -> np.ndarray:
    """Selected output blocks; returns float32 [nblk, 32, 32]."""
    A, B = _c(A, np.int8), _c(B, np.int8)
    sA, sB = _c(sA, np.float32), _c(sB, np.float32)
    blocks = np.ascontiguousarray(np.asarray(blocks, np.int64).reshape(-1, 2))
    M, N, K = _gemm_dims(ta, tb, A, B)
    out = np.empty((blocks.shape[0], 32, 32), np.float32)
    _chk(_load().jfo_gemm_f32_blocks(int(ta), int(tb), M, N, K, _p(A), _p(sA), _p(B), _p(sB),
                                      _p(blocks), blocks.shape[0], _p(out)), "gemm_f32_blocks")
    return out


def gemm_partial(A, B, I, J, kb, ta=0, tb=0) -> np.ndarray:
    """Exact int32 partial of output block (I, J) over k-block kb."""
    A, B = _c(A, np.int8), _c(B, np.int8)
    M, N, K = _gemm_dims(ta, tb, A, B)
    P = np.empty((32, 32), np.int32)
    _chk(_load().jfo_gemm_partial(int(ta), int(tb), M, N, K, _p(A), _p(B), I, J, kb, _p(P)), "gemm_partial")
    return P


def gemm_i8(A, sA, B, sB, ta=0, tb=0):
    """C = op(A) op(B), requantized per output block: (codes, scales)."""
    A, B = _c(A, np.int8), _c(B, np.int8)
    sA, sB = _c(sA, np.float32), _c(sB, np.float32)
    M, N, K = _gemm_dims(ta, tb, A, B)
    q = np.empty((M, N), np.int8)
    s = np.empty((M // 32, N // 32), np.float32)
    _chk(_load().jfo_gemm_i8(int(ta), int(tb), M, N, K, _p(A), _p(sA), _p(B), _p(sB), _p(q), _p(s)), "gemm_i8")
    return q, s


def gemm_i8_blocks(A, sA, B, sB, blocks, ta=0, tb=0):
    """Selected output blocks, requantized: (codes [nblk,32,32], scales [nblk])."""
    A, B = _c(A, np.int8), _c(B, np.int8)
    sA, sB = _c(sA, np.float32), _c(sB, np.float32)
    blocks = np.ascontiguousarray(np.asarray(blocks, np.int64).reshape(-1, 2))
    M, N, K = _gemm_dims(ta, tb, A, B)
    q = np.empty((blocks.shape[0], 32, 32), np.int8)
    s = np.empty((blocks.shape[0],), np.float32)
    _chk(_load().jfo_gemm_i8_blocks(int(ta), int(tb), M, N, K, _p(A), _p(sA), _p(B), _p(sB),
                                     _p(blocks), blocks.shape[0], _p(q), _p(s)), "gemm_i8_blocks")
    return q, s


def gelu_value(x: float) -> float:
    """g(x) = x * Phi(x) in binary64, rounded to binary32."""
    return float(_load().jfo_gelu_value(float(x)))


def gelu(q: np.ndarray, s: np.ndarray):
    """INT8 -> INT8 GELU with per-block requantization: (codes, scales)."""
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    R, C = q.shape
    qo = np.empty((R, C), np.int8)
    so = np.empty((R // 32, C // 32), np.float32)
    _chk(_load().jfo_gelu(_p(q), _p(s), R, C, _p(qo), _p(so)), "gelu")
    return qo, so


def gelu_grad_value(x: float) -> float:
    """GELU'(x) = Phi(x) + x phi(x) in binary64, rounded to binary32."""
    return float(_load().jfo_gelu_grad_value(float(x)))


def gelu_bwd(qdy: np.ndarray, sdy: np.ndarray, qx: np.ndarray, sx: np.ndarray):
    """INT8 GELU backward dX = dY * GELU'(X), requantized per block: (codes, scales)."""
    qdy, qx = _c(qdy, np.int8), _c(qx, np.int8)
    sdy, sx = _c(sdy, np.float32), _c(sx, np.float32)
    if qdy.shape != qx.shape or sdy.shape != sx.shape:
        raise ValueError("dY and X must have the same shape and blocking")
    R, C = qx.shape
    qo = np.empty((R, C), np.int8)
    so = np.empty((R // 32, C // 32), np.float32)
    _chk(_load().jfo_gelu_bwd(_p(qdy), _p(sdy), _p(qx), _p(sx), R, C, _p(qo), _p(so)), "gelu_bwd")
    return qo, so


def add(qa: np.ndarray, sa: np.ndarray, qb: np.ndarray, sb: np.ndarray):
    """Residual add of two per-block INT8 tensors with the same blocking,
    requantized per block: (codes, scales)."""
    qa, qb = _c(qa, np.int8), _c(qb, np.int8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    if qa.shape != qb.shape or sa.shape != sb.shape:
        raise ValueError("operands must have the same shape and blocking")
    R, C = qa.shape
    qo = np.empty((R, C), np.int8)
    so = np.empty((R // 32, C // 32), np.float32)
    _chk(_load().jfo_add(_p(qa), _p(sa), _p(qb), _p(sb), R, C, _p(qo), _p(so)), "add")
    return qo, so


def layernorm(q: np.ndarray, s: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = 1e-5,
              stats: bool = False):
    """LayerNorm over each row of a per-block INT8 tensor, requantized per
    block: (codes, scales), plus (mean, rstd) per row in binary64 if stats."""
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    gamma, beta = _c(gamma, np.float32), _c(beta, np.float32)
    R, C = q.shape
    if gamma.shape != (C,) or beta.shape != (C,):
        raise ValueError("gamma and beta must have one value per column")
    qo = np.empty((R, C), np.int8)
    so = np.empty((R // 32, C // 32), np.float32)
    mean = np.empty(R, np.float64)
    rstd = np.empty(R, np.float64)
    _chk(_load().jfo_layernorm(_p(q), _p(s), R, C, _p(gamma), _p(beta), float(np.float32(eps)), _p(qo), _p(so),
                               _p(mean), _p(rstd)), "layernorm")
    return (qo, so, mean, rstd) if stats else (qo, so)


GRANULARITIES = {"block": 0, "token": 1, "channel": 2, "tensor": 3}


def quant_sse(x: np.ndarray, granularity: str):
    """Scales and sum of squared quantization errors for one scale granularity
    ('block' 32x32, 'token' per row, 'channel' per column, 'tensor')."""
    x = _c(x, np.float32)
    R, C = x.shape
    g = GRANULARITIES[granularity]
    s = np.empty(int(_load().jfo_quant_groups(g, R, C)), np.float32)
    sse = np.zeros(1, np.float64)
    _chk(_load().jfo_quant_sse(_p(x), R, C, g, _p(s), _p(sse)), "quant_sse")
    return s, float(sse[0])
