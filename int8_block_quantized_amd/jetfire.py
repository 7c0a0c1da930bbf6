"""ctypes binding of libjetfire.so (C ABI in include/jetfire.h).

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI.  torch supplies device memory (outputs are allocated with
``torch.empty`` on the input's device) and the stream (the device's current
stream).  There is no fallback: if the library is missing, importing this
module raises.

Names follow the C ABI:  quantize_block, dequantize_block, gemm_i8_blockscaled,
requant_block, gelu_i8, gelu_bwd_i8, add_i8, layernorm_i8, quant_error.  A tensor argument is a 2-D CUDA(HIP) tensor whose last dimension is
contiguous; its row stride is passed as the leading dimension.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libjetfire.so")

JF_OK, JF_ERR_NULL, JF_ERR_SHAPE, JF_ERR_LD, JF_ERR_ALIGN = 0, 1, 2, 3, 4
JF_ERR_DTYPE, JF_ERR_ARG, JF_ERR_ALIAS, JF_ERR_HIP = 5, 6, 7, 8
JF_F32, JF_BF16 = 0, 1
JF_OUT_I8, JF_OUT_F32 = 0, 1
GRANULARITIES = {"block": 0, "token": 1, "channel": 2, "tensor": 3}

# Every symbol include/jetfire.h declares.
EXPORTS = ("jf_quantize_block", "jf_dequantize_block", "jf_gemm_i8_blockscaled", "jf_requant_block", "jf_gelu_i8",
           "jf_gelu_bwd_i8", "jf_add_i8", "jf_layernorm_i8", "jf_quant_error", "jf_status_str",
           "jf_abi_version")


class JetfireError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    i64, ptr, cint = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.jf_quantize_block.argtypes = [cint, ptr, i64, i64, i64, ptr, i64, ptr, ptr]
    lib.jf_quantize_block.restype = cint
    lib.jf_requant_block.argtypes = [ptr, i64, i64, i64, ptr, i64, ptr, ptr]
    lib.jf_requant_block.restype = cint
    lib.jf_dequantize_block.argtypes = [ptr, i64, ptr, i64, i64, cint, ptr, i64, ptr]
    lib.jf_dequantize_block.restype = cint
    lib.jf_gemm_i8_blockscaled.argtypes = [cint, cint, i64, i64, i64, ptr, i64, ptr, ptr, i64, ptr,
                                           cint, ptr, i64, ptr, ptr]
    lib.jf_gemm_i8_blockscaled.restype = cint
    lib.jf_gelu_i8.argtypes = [ptr, i64, ptr, i64, i64, ptr, i64, ptr, ptr]
    lib.jf_gelu_i8.restype = cint
    lib.jf_gelu_bwd_i8.argtypes = [ptr, i64, ptr, ptr, i64, ptr, i64, i64, ptr, i64, ptr, ptr]
    lib.jf_gelu_bwd_i8.restype = cint
    lib.jf_add_i8.argtypes = [ptr, i64, ptr, ptr, i64, ptr, i64, i64, ptr, i64, ptr, ptr]
    lib.jf_add_i8.restype = cint
    lib.jf_layernorm_i8.argtypes = [ptr, i64, ptr, i64, i64, ptr, ptr, ctypes.c_float, ptr, i64, ptr, ptr, ptr,
                                    ptr]
    lib.jf_layernorm_i8.restype = cint
    lib.jf_quant_error.argtypes = [ptr, i64, i64, i64, cint, ptr, ptr, ptr]
    lib.jf_quant_error.restype = cint
    lib.jf_status_str.argtypes = [cint]
    lib.jf_status_str.restype = ctypes.c_char_p
    lib.jf_abi_version.restype = cint
    return lib


lib = _load()


def status_str(status: int) -> str:
    return lib.jf_status_str(int(status)).decode()


def abi_version() -> int:
    return int(lib.jf_abi_version())


def _check(status: int, where: str) -> None:
    if status != JF_OK:
        raise JetfireError(status, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _mat(t: torch.Tensor, name: str) -> int:
    """Validate a 2-D device matrix with a contiguous last dimension and
    return its leading dimension (row stride in elements)."""
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (the HIP path has no CPU fallback)")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")
    # an empty or one-row matrix has no meaningful row stride: pass the row length
    return int(t.stride(0)) if t.shape[0] > 1 and t.numel() > 0 else int(t.shape[1])


def _scales(t: torch.Tensor, rows: int, cols: int, name: str) -> None:
    if t.dtype != torch.float32 or not t.is_cuda or tuple(t.shape) != (rows // 32, cols // 32) \
            or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 device tensor of shape "
                         f"({rows // 32}, {cols // 32})")


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def quantize_block(x: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None):
    """jf_quantize_block: float32/bfloat16 [R, C] -> (int8 codes [R, C],
    float32 scales [R/32, C/32])."""
    ldx = _mat(x, "x")
    if x.dtype == torch.float32:
        xt = JF_F32
    elif x.dtype == torch.bfloat16:
        xt = JF_BF16
    else:
        raise ValueError("x must be float32 or bfloat16")
    R, C = x.shape
    q = torch.empty((R, C), dtype=torch.int8, device=x.device) if q is None else q
    s = torch.empty((R // 32, C // 32), dtype=torch.float32, device=x.device) if s is None else s
    ldq = _mat(q, "q")
    _check(lib.jf_quantize_block(xt, _ptr(x), ldx, R, C, _ptr(q), ldq, _ptr(s), _stream(x.device)),
           "jf_quantize_block")
    return q, s


def requant_block(x: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None):
    """jf_requant_block: float32 [R, C] -> (int8 codes, float32 scales)."""
    ldx = _mat(x, "x")
    if x.dtype != torch.float32:
        raise ValueError("x must be float32")
    R, C = x.shape
    q = torch.empty((R, C), dtype=torch.int8, device=x.device) if q is None else q
    s = torch.empty((R // 32, C // 32), dtype=torch.float32, device=x.device) if s is None else s
    ldq = _mat(q, "q")
    _check(lib.jf_requant_block(_ptr(x), ldx, R, C, _ptr(q), ldq, _ptr(s), _stream(x.device)),
           "jf_requant_block")
    return q, s


def dequantize_block(q: torch.Tensor, s: torch.Tensor, dtype: torch.dtype = torch.float32,
                     y: torch.Tensor | None = None) -> torch.Tensor:
    """jf_dequantize_block: int8 codes [R, C] + float32 scales [R/32, C/32]
    -> float32 fl(s*q), or that value rounded to bfloat16 (``dtype``)."""
    ldq = _mat(q, "q")
    if q.dtype != torch.int8:
        raise ValueError("q must be int8")
    if dtype == torch.float32:
        yt = JF_F32
    elif dtype == torch.bfloat16:
        yt = JF_BF16
    else:
        raise ValueError("dtype must be float32 or bfloat16")
    R, C = q.shape
    _scales(s, R, C, "s")
    y = torch.empty((R, C), dtype=dtype, device=q.device) if y is None else y
    if y.dtype != dtype:
        raise ValueError("y must have the requested dtype")
    ldy = _mat(y, "y")
    _check(lib.jf_dequantize_block(_ptr(q), ldq, _ptr(s), R, C, yt, _ptr(y), ldy, _stream(q.device)),
           "jf_dequantize_block")
    return y


def gemm_i8_blockscaled(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
                        trans_a: bool = False, trans_b: bool = False, out: str = "i8",
                        c: torch.Tensor | None = None, sc: torch.Tensor | None = None):
    """jf_gemm_i8_blockscaled: C = op(a) op(b).  ``a`` is stored M x K
    (trans_a False) or K x M; ``b`` is stored K x N (trans_b False) or N x K;
    ``sa``/``sb`` are their scale grids in stored orientation.  ``out="i8"``
    returns (codes int8 [M, N], scales float32 [M/32, N/32]); ``out="f32"``
    returns float32 [M, N]."""
    lda, ldb = _mat(a, "a"), _mat(b, "b")
    if a.dtype != torch.int8 or b.dtype != torch.int8:
        raise ValueError("a and b must be int8 codes")
    M, K = (a.shape[1], a.shape[0]) if trans_a else (a.shape[0], a.shape[1])
    Kb, N = (b.shape[1], b.shape[0]) if trans_b else (b.shape[0], b.shape[1])
    if K != Kb:
        raise ValueError(f"inner dimensions differ: {K} vs {Kb}")
    _scales(sa, a.shape[0], a.shape[1], "sa")
    _scales(sb, b.shape[0], b.shape[1], "sb")
    dev = a.device
    if out == "i8":
        c = torch.empty((M, N), dtype=torch.int8, device=dev) if c is None else c
        sc = torch.empty((M // 32, N // 32), dtype=torch.float32, device=dev) if sc is None else sc
        kind = JF_OUT_I8
    elif out == "f32":
        c = torch.empty((M, N), dtype=torch.float32, device=dev) if c is None else c
        sc = None
        kind = JF_OUT_F32
    else:
        raise ValueError("out must be 'i8' or 'f32'")
    ldc = _mat(c, "c")
    _check(lib.jf_gemm_i8_blockscaled(int(trans_a), int(trans_b), M, N, K, _ptr(a), lda, _ptr(sa),
                                      _ptr(b), ldb, _ptr(sb), kind, _ptr(c), ldc, _ptr(sc), _stream(dev)),
           "jf_gemm_i8_blockscaled")
    return (c, sc) if out == "i8" else c


def gelu_i8(q: torch.Tensor, s: torch.Tensor, qo: torch.Tensor | None = None,
            so: torch.Tensor | None = None):
    """jf_gelu_i8: INT8 codes + scales -> GELU, requantized per block."""
    ldq = _mat(q, "q")
    if q.dtype != torch.int8:
        raise ValueError("q must be int8")
    R, C = q.shape
    _scales(s, R, C, "s")
    qo = torch.empty((R, C), dtype=torch.int8, device=q.device) if qo is None else qo
    so = torch.empty((R // 32, C // 32), dtype=torch.float32, device=q.device) if so is None else so
    ldqo = _mat(qo, "qo")
    _check(lib.jf_gelu_i8(_ptr(q), ldq, _ptr(s), R, C, _ptr(qo), ldqo, _ptr(so), _stream(q.device)),
           "jf_gelu_i8")
    return qo, so


def gelu_bwd_i8(qdy: torch.Tensor, sdy: torch.Tensor, qx: torch.Tensor, sx: torch.Tensor,
                qo: torch.Tensor | None = None, so: torch.Tensor | None = None):
    """jf_gelu_bwd_i8: dX = dY * GELU'(X) on INT8 codes + scales, requantized per block."""
    lddy, ldx = _mat(qdy, "qdy"), _mat(qx, "qx")
    if qdy.dtype != torch.int8 or qx.dtype != torch.int8:
        raise ValueError("qdy and qx must be int8")
    if qdy.shape != qx.shape:
        raise ValueError("qdy and qx must have the same shape")
    R, C = qx.shape
    _scales(sdy, R, C, "sdy")
    _scales(sx, R, C, "sx")
    qo = torch.empty((R, C), dtype=torch.int8, device=qx.device) if qo is None else qo
    so = torch.empty((R // 32, C // 32), dtype=torch.float32, device=qx.device) if so is None else so
    ldo = _mat(qo, "qo")
    _check(lib.jf_gelu_bwd_i8(_ptr(qdy), lddy, _ptr(sdy), _ptr(qx), ldx, _ptr(sx), R, C, _ptr(qo), ldo, _ptr(so),
                              _stream(qx.device)), "jf_gelu_bwd_i8")
    return qo, so


def add_i8(qa: torch.Tensor, sa: torch.Tensor, qb: torch.Tensor, sb: torch.Tensor,
           qo: torch.Tensor | None = None, so: torch.Tensor | None = None):
    """jf_add_i8: residual add of two per-block INT8 tensors, requantized per block."""
    lda, ldb = _mat(qa, "qa"), _mat(qb, "qb")
    if qa.dtype != torch.int8 or qb.dtype != torch.int8:
        raise ValueError("qa and qb must be int8")
    if qa.shape != qb.shape:
        raise ValueError("qa and qb must have the same shape")
    R, C = qa.shape
    _scales(sa, R, C, "sa")
    _scales(sb, R, C, "sb")
    qo = torch.empty((R, C), dtype=torch.int8, device=qa.device) if qo is None else qo
    so = torch.empty((R // 32, C // 32), dtype=torch.float32, device=qa.device) if so is None else so
    ldo = _mat(qo, "qo")
    _check(lib.jf_add_i8(_ptr(qa), lda, _ptr(sa), _ptr(qb), ldb, _ptr(sb), R, C, _ptr(qo), ldo, _ptr(so),
                         _stream(qa.device)), "jf_add_i8")
    return qo, so


def layernorm_i8(q: torch.Tensor, s: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, eps: float = 1e-5,
                 qo: torch.Tensor | None = None, so: torch.Tensor | None = None, stats: bool = False):
    """jf_layernorm_i8: LayerNorm over each row of per-block INT8 codes, INT8 out.
    Returns (qo, so), or (qo, so, mean, rstd) with float64 row statistics if stats."""
    ldq = _mat(q, "q")
    if q.dtype != torch.int8:
        raise ValueError("q must be int8")
    R, C = q.shape
    _scales(s, R, C, "s")
    for t, n in ((gamma, "gamma"), (beta, "beta")):
        if t.dtype != torch.float32 or not t.is_cuda or tuple(t.shape) != (C,) or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous float32 device tensor of shape ({C},)")
    qo = torch.empty((R, C), dtype=torch.int8, device=q.device) if qo is None else qo
    so = torch.empty((R // 32, C // 32), dtype=torch.float32, device=q.device) if so is None else so
    ldo = _mat(qo, "qo")
    mean = torch.empty(R, dtype=torch.float64, device=q.device) if stats else None
    rstd = torch.empty(R, dtype=torch.float64, device=q.device) if stats else None
    _check(lib.jf_layernorm_i8(_ptr(q), ldq, _ptr(s), R, C, _ptr(gamma), _ptr(beta), float(eps), _ptr(qo), ldo,
                               _ptr(so), _ptr(mean), _ptr(rstd), _stream(q.device)), "jf_layernorm_i8")
    return (qo, so, mean, rstd) if stats else (qo, so)


def scale_count(granularity: str, rows: int, cols: int) -> int:
    g = GRANULARITIES[granularity]
    return (rows // 32) * (cols // 32) if g == 0 else rows if g == 1 else cols if g == 2 else 1


def quant_error(x: torch.Tensor, granularity: str, s: torch.Tensor | None = None,
                sse: torch.Tensor | None = None):
    """jf_quant_error: group scales (1-D float32) and the binary64 sum of squared
    quantization errors (1-element float64 tensor) of a float32 matrix under
    'block' (32x32), 'token', 'channel' or 'tensor' scaling."""
    ldx = _mat(x, "x")
    if x.dtype != torch.float32:
        raise ValueError("x must be float32")
    if granularity not in GRANULARITIES:
        raise ValueError(f"granularity must be one of {sorted(GRANULARITIES)}")
    R, C = x.shape
    n = scale_count(granularity, R, C)
    s = torch.empty(n, dtype=torch.float32, device=x.device) if s is None else s
    sse = torch.empty(1, dtype=torch.float64, device=x.device) if sse is None else sse
    if s.dtype != torch.float32 or not s.is_cuda or s.numel() != n or not s.is_contiguous():
        raise ValueError(f"s must be a contiguous float32 device tensor of {n} elements")
    if sse.dtype != torch.float64 or not sse.is_cuda or sse.numel() != 1:
        raise ValueError("sse must be a one-element float64 device tensor")
    _check(lib.jf_quant_error(_ptr(x), ldx, R, C, GRANULARITIES[granularity], _ptr(s), _ptr(sse),
                              _stream(x.device)), "jf_quant_error")
    return s, sse
