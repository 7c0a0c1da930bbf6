"""C ABI host logic, without a GPU.

The library must load, export every symbol include/jetfire.h declares, and
reject bad arguments with the documented status codes BEFORE any HIP call
(the header promises validation first), so every case here returns without
touching a device.  Pointers below are fake addresses; none is dereferenced.
"""
import ctypes
import os
import re

import pytest

from int8_block_quantized_amd import jetfire as jf

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "jetfire.h")

P = ctypes.c_void_p
BASE = 0x7f0000000000          # fake, 256-byte aligned addresses
A_, B_, SA, SB, C_, SC = (P(BASE + i * 0x10000000) for i in range(6))


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"JF_API\s+[\w\s\*]+?\b(jf_\w+)\s*\(", text)


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert set(names) == set(jf.EXPORTS)
    for n in names:
        assert hasattr(jf.lib, n), n


def test_version_and_status_strings():
    assert jf.abi_version() == 5
    for st in range(0, 9):
        assert jf.status_str(st) and jf.status_str(st) != "unknown status"
    assert jf.status_str(99) == "unknown status"


def gemm(ta=0, tb=0, M=64, N=64, K=64, A=A_, lda=None, sA=SA, B=B_, ldb=None, sB=SB, out=jf.JF_OUT_I8,
         C=C_, ldc=None, sC=SC):
    lda = lda if lda is not None else (M if ta else K)
    ldb = ldb if ldb is not None else (K if tb else N)
    ldc = ldc if ldc is not None else N
    return jf.lib.jf_gemm_i8_blockscaled(ta, tb, M, N, K, A, lda, sA, B, ldb, sB, out, C, ldc, sC, None)


def test_gemm_validation_codes():
    assert gemm(A=None) == jf.JF_ERR_NULL
    assert gemm(sB=None) == jf.JF_ERR_NULL
    assert gemm(sC=None) == jf.JF_ERR_NULL                      # required for INT8 output
    assert gemm(M=0, A=None, C=None, sC=None) == jf.JF_OK        # empty output: nothing to do
    assert gemm(M=48) == jf.JF_ERR_SHAPE
    assert gemm(K=-32) == jf.JF_ERR_SHAPE
    assert gemm(out=7) == jf.JF_ERR_DTYPE
    assert gemm(ta=2) == jf.JF_ERR_ARG
    assert gemm(tb=-1) == jf.JF_ERR_ARG
    assert gemm(lda=32) == jf.JF_ERR_LD                          # below the row length
    assert gemm(ldb=72) == jf.JF_ERR_LD                          # pitch not 16-byte multiple
    assert gemm(out=jf.JF_OUT_F32, ldc=66, sC=None) == jf.JF_ERR_LD   # 264-byte pitch
    assert gemm(A=P(BASE + 8)) == jf.JF_ERR_ALIGN
    assert gemm(sA=P(BASE + 0x10000002)) == jf.JF_ERR_ALIGN
    # output codes overlapping the A operand
    assert gemm(C=P(BASE + 0x100)) == jf.JF_ERR_ALIAS
    # output scales overlapping the output codes
    assert gemm(sC=P(BASE + 4 * 0x10000000 + 64)) == jf.JF_ERR_ALIAS


def test_quantize_validation_codes():
    q = jf.lib.jf_quantize_block
    x, qq, s = P(BASE), P(BASE + 0x10000000), P(BASE + 0x20000000)
    assert q(jf.JF_F32, None, 64, 64, 64, qq, 64, s, None) == jf.JF_ERR_NULL
    assert q(jf.JF_F32, x, 64, 64, 40, qq, 64, s, None) == jf.JF_ERR_SHAPE
    assert q(3, x, 64, 64, 64, qq, 64, s, None) == jf.JF_ERR_DTYPE
    assert q(jf.JF_F32, x, 32, 64, 64, qq, 64, s, None) == jf.JF_ERR_LD
    assert q(jf.JF_BF16, x, 68, 64, 64, qq, 64, s, None) == jf.JF_ERR_LD    # 136 B pitch
    assert q(jf.JF_F32, x, 64, 64, 64, qq, 72, s, None) == jf.JF_ERR_LD     # 72 B pitch
    assert q(jf.JF_F32, P(BASE + 4), 64, 64, 64, qq, 64, s, None) == jf.JF_ERR_ALIGN
    assert q(jf.JF_F32, x, 64, 64, 64, qq, 64, P(BASE + 0x20000002), None) == jf.JF_ERR_ALIGN
    assert q(jf.JF_F32, x, 64, 64, 64, P(BASE + 1024), 64, s, None) == jf.JF_ERR_ALIAS
    # empty input: valid, nothing launched, NULL allowed
    assert q(jf.JF_F32, x, 64, 0, 64, qq, 64, s, None) == jf.JF_OK
    assert q(jf.JF_F32, None, 64, 0, 64, None, 64, None, None) == jf.JF_OK
    r = jf.lib.jf_requant_block
    assert r(None, 64, 64, 64, qq, 64, s, None) == jf.JF_ERR_NULL
    assert r(x, 64, 64, 64, qq, 64, P(BASE + 0x40), None) == jf.JF_ERR_ALIAS


def test_dequantize_validation_codes():
    d = jf.lib.jf_dequantize_block
    q, s, y = P(BASE), P(BASE + 0x10000000), P(BASE + 0x20000000)
    assert d(q, 64, None, 64, 64, jf.JF_F32, y, 64, None) == jf.JF_ERR_NULL
    assert d(q, 64, s, 64, 64, jf.JF_BF16, None, 64, None) == jf.JF_ERR_NULL
    assert d(q, 64, s, 72, 64, jf.JF_F32, y, 64, None) == jf.JF_ERR_SHAPE
    assert d(q, 64, s, 64, 64, 2, y, 64, None) == jf.JF_ERR_DTYPE
    assert d(q, 48, s, 64, 64, jf.JF_F32, y, 64, None) == jf.JF_ERR_LD            # below the row length
    assert d(q, 64, s, 64, 64, jf.JF_F32, y, 66, None) == jf.JF_ERR_LD            # 264-byte pitch
    assert d(q, 64, s, 64, 64, jf.JF_BF16, y, 68, None) == jf.JF_ERR_LD           # 136-byte pitch
    assert d(P(BASE + 8), 64, s, 64, 64, jf.JF_F32, y, 64, None) == jf.JF_ERR_ALIGN
    assert d(q, 64, s, 64, 64, jf.JF_F32, P(BASE + 0x20000008), 64, None) == jf.JF_ERR_ALIGN
    assert d(q, 64, P(BASE + 0x10000002), 64, 64, jf.JF_F32, y, 64, None) == jf.JF_ERR_ALIGN
    assert d(q, 64, s, 64, 64, jf.JF_F32, P(BASE + 0x100), 64, None) == jf.JF_ERR_ALIAS     # over the codes
    assert d(q, 64, s, 64, 64, jf.JF_BF16, P(BASE + 0x10000000 - 8192 + 16), 64, None) == jf.JF_ERR_ALIAS  # over s
    assert d(q, 64, s, 0, 64, jf.JF_F32, None, 64, None) == jf.JF_OK                # empty


def test_gelu_validation_codes():
    g = jf.lib.jf_gelu_i8
    q, s, qo, so = P(BASE), P(BASE + 0x10000000), P(BASE + 0x20000000), P(BASE + 0x30000000)
    assert g(q, 64, s, 64, 64, None, 64, so, None) == jf.JF_ERR_NULL
    assert g(q, 64, s, 64, 96 + 8, qo, 64, so, None) == jf.JF_ERR_SHAPE
    assert g(q, 64, s, 64, 64, qo, 48, so, None) == jf.JF_ERR_LD
    assert g(q, 64, s, 64, 64, P(BASE + 0x20000008), 64, so, None) == jf.JF_ERR_ALIGN
    assert g(q, 64, s, 64, 64, q, 64, so, None) == jf.JF_ERR_ALIAS           # in place
    assert g(q, 64, s, 64, 64, qo, 64, s, None) == jf.JF_ERR_ALIAS
    assert g(q, 64, s, 0, 64, qo, 64, so, None) == jf.JF_OK                  # empty


def test_gelu_bwd_validation_codes():
    g = jf.lib.jf_gelu_bwd_i8
    dy, sdy, x, sx = P(BASE), P(BASE + 0x10000000), P(BASE + 0x20000000), P(BASE + 0x30000000)
    qo, so = P(BASE + 0x40000000), P(BASE + 0x50000000)
    assert g(dy, 64, sdy, None, 64, sx, 64, 64, qo, 64, so, None) == jf.JF_ERR_NULL
    assert g(dy, 64, sdy, x, 64, sx, 64, 80, qo, 64, so, None) == jf.JF_ERR_SHAPE
    assert g(dy, 64, sdy, x, 32, sx, 64, 64, qo, 64, so, None) == jf.JF_ERR_LD
    assert g(dy, 64, sdy, x, 64, sx, 64, 64, qo, 72, so, None) == jf.JF_ERR_LD
    assert g(dy, 64, sdy, x, 64, P(BASE + 0x30000002), 64, 64, qo, 64, so, None) == jf.JF_ERR_ALIGN
    assert g(dy, 64, sdy, x, 64, sx, 64, 64, dy, 64, so, None) == jf.JF_ERR_ALIAS     # over dY
    assert g(dy, 64, sdy, x, 64, sx, 64, 64, P(BASE + 0x20000100), 64, so, None) == jf.JF_ERR_ALIAS
    assert g(dy, 64, sdy, x, 64, sx, 64, 64, qo, 64, sx, None) == jf.JF_ERR_ALIAS
    assert g(dy, 64, sdy, x, 64, sx, 0, 64, qo, 64, so, None) == jf.JF_OK             # empty


def test_add_validation_codes():
    f = jf.lib.jf_add_i8
    a, sa, b, sb = P(BASE), P(BASE + 0x10000000), P(BASE + 0x20000000), P(BASE + 0x30000000)
    qo, so = P(BASE + 0x40000000), P(BASE + 0x50000000)
    assert f(a, 64, sa, None, 64, sb, 64, 64, qo, 64, so, None) == jf.JF_ERR_NULL
    assert f(a, 64, sa, b, 64, sb, 64, 64, qo, 64, None, None) == jf.JF_ERR_NULL
    assert f(a, 64, sa, b, 64, sb, 40, 64, qo, 64, so, None) == jf.JF_ERR_SHAPE
    assert f(a, 64, sa, b, 32, sb, 64, 64, qo, 64, so, None) == jf.JF_ERR_LD
    assert f(a, 64, sa, b, 64, sb, 64, 64, qo, 68, so, None) == jf.JF_ERR_LD
    assert f(P(BASE + 8), 64, sa, b, 64, sb, 64, 64, qo, 64, so, None) == jf.JF_ERR_ALIGN
    assert f(a, 64, sa, b, 64, P(BASE + 0x30000001), 64, 64, qo, 64, so, None) == jf.JF_ERR_ALIGN
    assert f(a, 64, sa, b, 64, sb, 64, 64, a, 64, so, None) == jf.JF_ERR_ALIAS          # in place
    assert f(a, 64, sa, b, 64, sb, 64, 64, qo, 64, P(BASE + 0x20000000 + 4032), None) == jf.JF_ERR_ALIAS
    assert f(a, 64, sa, b, 64, sb, 64, 64, qo, 64, P(BASE + 0x40000000 + 4080), None) == jf.JF_ERR_ALIAS
    assert f(a, 64, sa, b, 64, sb, 0, 64, None, 64, None, None) == jf.JF_OK                # empty


def test_layernorm_validation_codes():
    f = jf.lib.jf_layernorm_i8
    q, s, g, b = P(BASE), P(BASE + 0x10000000), P(BASE + 0x20000000), P(BASE + 0x30000000)
    qo, so, m, r = P(BASE + 0x40000000), P(BASE + 0x50000000), P(BASE + 0x60000000), P(BASE + 0x70000000)

    def ln(q=q, ldq=64, s=s, rows=64, cols=64, g=g, b=b, eps=1e-5, qo=qo, ldo=64, so=so, m=m, r=r):
        return f(q, ldq, s, rows, cols, g, b, eps, qo, ldo, so, m, r, None)

    assert ln(g=None) == jf.JF_ERR_NULL
    assert ln(so=None) == jf.JF_ERR_NULL
    assert ln(cols=80) == jf.JF_ERR_SHAPE
    assert ln(ldq=48) == jf.JF_ERR_LD
    assert ln(b=P(BASE + 0x30000004)) == jf.JF_ERR_ALIGN                  # beta is read 16 bytes at a time
    assert ln(m=P(BASE + 0x60000004)) == jf.JF_ERR_ALIGN
    assert ln(eps=-1e-6) == jf.JF_ERR_ARG
    assert ln(eps=float("inf")) == jf.JF_ERR_ARG
    assert ln(eps=float("nan")) == jf.JF_ERR_ARG
    assert ln(qo=q) == jf.JF_ERR_ALIAS
    assert ln(m=P(BASE + 0x20000000 + 128)) == jf.JF_ERR_ALIAS             # mean over gamma
    assert ln(r=P(BASE + 0x60000000 + 256)) == jf.JF_ERR_ALIAS             # rstd over mean
    assert ln(rows=0, q=None, s=None, qo=None, so=None) == jf.JF_OK


def test_quant_error_validation_codes():
    q = jf.lib.jf_quant_error
    x, s, e = P(BASE), P(BASE + 0x10000000), P(BASE + 0x20000000)
    assert q(None, 64, 64, 64, 0, s, e, None) == jf.JF_ERR_NULL
    assert q(x, 64, 64, 64, 0, s, None, None) == jf.JF_ERR_NULL          # the sum is always required
    assert q(x, 64, 64, 64, 3, None, e, None) == jf.JF_ERR_NULL          # one tensor scale even if empty
    assert q(x, 64, 64, 64, 9, None, e, None) == jf.JF_ERR_NULL          # unknown granularity: s required
    assert q(x, 64, 64, 48, 0, s, e, None) == jf.JF_ERR_SHAPE
    assert q(x, 64, -32, 64, 1, s, e, None) == jf.JF_ERR_SHAPE
    assert q(x, 32, 64, 64, 0, s, e, None) == jf.JF_ERR_LD               # below the row length
    assert q(x, 66, 64, 64, 0, s, e, None) == jf.JF_ERR_LD               # 264-byte pitch
    assert q(P(BASE + 4), 64, 64, 64, 0, s, e, None) == jf.JF_ERR_ALIGN
    assert q(x, 64, 64, 64, 0, P(BASE + 0x10000002), e, None) == jf.JF_ERR_ALIGN
    assert q(x, 64, 64, 64, 0, s, P(BASE + 0x20000004), None) == jf.JF_ERR_ALIGN
    assert q(x, 64, 64, 64, 4, s, e, None) == jf.JF_ERR_ARG
    assert q(x, 64, 64, 64, -1, s, e, None) == jf.JF_ERR_ARG
    assert q(x, 64, 64, 64, 1, P(BASE + 64 * 64 * 4 - 4), e, None) == jf.JF_ERR_ALIAS   # s over x's last row
    assert q(x, 64, 64, 64, 2, s, P(BASE + 0x10000000 + 4 * 62), None) == jf.JF_ERR_ALIAS  # sse over s


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        jf.quantize_block(torch.zeros(32, 32))


def test_binding_fails_loudly_without_the_library(tmp_path, monkeypatch):
    """No fallback: with libjetfire.so absent the binding's loader raises
    instead of handing out another implementation."""
    monkeypatch.setattr(jf, "LIB_PATH", str(tmp_path / "libjetfire.so"))
    with pytest.raises(ImportError, match="not built"):
        jf._load()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus above 1 exits with a message before
    touching a device."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and not res.stdout.strip()
