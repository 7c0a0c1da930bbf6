"""Helpers for the GPU parity tests: device transfer and the parity bars.

Bars (per the method's contract as read for this library):
  * quantize: codes and scales bit-exact;
  * GEMM int32 partials: bit-exact;
  * GEMM binary32 output: |gpu - oracle| <= 1e-5 * sum_k |sigma_k P_k| per
    element and ||gpu - oracle||_F <= 1e-5 ||oracle||_F;
  * requantized INT8 (GEMM epilogue, GELU): codes within 1 LSB on at most
    0.01% of elements, scales within 1e-6 relative.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = torch.device("cuda:0")


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_requant_close(q, s, ref_q, ref_s, what="", max_frac=1e-4, s_rtol=1e-6):
    q = np.asarray(q).astype(np.int32)
    ref_q = np.asarray(ref_q).astype(np.int32)
    d = np.abs(q - ref_q)
    frac = float((d > 0).mean()) if d.size else 0.0
    assert d.max(initial=0) <= 1, f"{what}: code differs by {d.max()}"
    assert frac <= max_frac, f"{what}: {frac:.2e} of codes differ"
    s, ref_s = np.asarray(s, np.float64), np.asarray(ref_s, np.float64)
    zero = ref_s == 0
    assert np.all(s[zero] == 0), f"{what}: non-zero scale where the oracle has 0"
    rel = np.abs(s[~zero] - ref_s[~zero]) / ref_s[~zero]
    assert rel.max(initial=0) <= s_rtol, f"{what}: scale rel err {rel.max():.2e}"
    return frac, float(rel.max(initial=0))


def block_abs_terms(A_log: np.ndarray, sA_log: np.ndarray, B_log: np.ndarray, sB_log: np.ndarray,
                    I: int, J: int) -> np.ndarray:
    """sum_k |sigma_k P_k| for output block (I, J), float64 (32 x 32)."""
    K = A_log.shape[1]
    nk = K // 32
    a = A_log[32 * I:32 * I + 32, :].astype(np.int64).reshape(32, nk, 32).transpose(1, 0, 2)
    b = B_log[:, 32 * J:32 * J + 32].astype(np.int64).reshape(nk, 32, 32)
    P = np.matmul(a, b)                                      # (nk, 32, 32) exact
    sig = sA_log[I, :].astype(np.float64) * sB_log[:, J].astype(np.float64)
    return np.abs(P * sig[:, None, None]).sum(0)


def assert_f32_close(got, ref, absterm, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= 1e-5 * absterm + 1e-37), f"{what}: elementwise bound exceeded ({(err / (absterm + 1e-37)).max():.2e})"
    nr = np.linalg.norm(ref)
    if nr > 0:
        assert np.linalg.norm(got - ref) <= 1e-5 * nr, f"{what}: normwise bound exceeded"
    return float((err == 0).mean())
