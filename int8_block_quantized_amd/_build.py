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


# exhaustive checks of the GELU kernels' elementary-function evaluations,
# run by the GPU tests
TEST_PROBES = ("gelu_bound_check", "gelu_grad_check")


def build_test_probe(verbose: bool = False) -> list:
    """Compile the exhaustive GELU / GELU' checks used by the GPU tests."""
    built = []
    for name in TEST_PROBES:
        src, out = os.path.join(ROOT, "tests", name + ".hip"), os.path.join(ROOT, "tests", name)
        tmp = out + ".tmp"
        cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed:\n{res.stdout}\n{res.stderr}")
        os.replace(tmp, out)
        built.append(out)
    return built


# Extra flags for single sources (machine-scheduler settings, each measured
# against the alternative on the same MI355X): gemm.hip max-ILP (+1% on the
# hidden-4096 GEMMs) with the AMDGPU register-pressure trackers (+0.9% more),
# quantize.hip max-memory-clause (+1.5% on 16384^2).
# Neither is library-wide: max-ILP makes the GELU kernels 14-15% slower,
# max-memory-clause the GELU backward 8% and the residual add 20%.
PER_SOURCE_FLAGS = {
    "gemm.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp", "-mllvm", "-amdgpu-use-amdgpu-trackers=true"],
    "quantize.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
}


CEIL_SRC = os.path.join(PKG, "ceilings", "ceilings.hip")
CEIL_PATH = os.path.join(PKG, "libjfceil.so")


def build_ceilings(verbose: bool = False) -> str:
    """Compile the benchmark's measured-ceiling kernels (register-only MFMA
    loops, streaming copies) into libjfceil.so.  Not part of the hot path."""
    tmp = CEIL_PATH + ".tmp"
    cmd = ["hipcc", *HIPCC_FLAGS, CEIL_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, CEIL_PATH)
    return CEIL_PATH


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libjetfire.so (always recompiles): one
    object per source (in parallel), then one shared-library link."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    procs = []
    for src in sources():
        name = os.path.basename(src)
        obj = os.path.join(objdir, name + ".o")
        cmd = ["hipcc", *compile_flags, *PER_SOURCE_FLAGS.get(name, []), "-I", os.path.join(ROOT, "include"),
               "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    objs = []
    for cmd, obj, pr in procs:
        out, err = pr.communicate()
        if pr.returncode != 0:
            raise RuntimeError(f"hipcc failed: {' '.join(cmd)}\n{out}\n{err}")
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH
