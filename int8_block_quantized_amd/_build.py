"""Build of libjetfire.so (HIP, gfx950 only) in-tree, next to this file."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libjetfire.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # every rounding in the kernels is written explicitly (fmaf where fused)
    "-ffp-contract=off",
    # no packed binary32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in architectural VGPRs: the per-k-block rescale reads them
    # with VALU instructions, and an AGPR destination would cost one extra
    # v_accvgpr_read per element
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


TEST_PROBE_SRC = os.path.join(ROOT, "tests", "gelu_bound_check.hip")
TEST_PROBE_BIN = os.path.join(ROOT, "tests", "gelu_bound_check")


def build_test_probe(verbose: bool = False) -> str:
    """Compile the exhaustive GELU error check used by the GPU tests."""
    tmp = TEST_PROBE_BIN + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", TEST_PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, TEST_PROBE_BIN)
    return TEST_PROBE_BIN


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libjetfire.so (always recompiles)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["hipcc", *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH
