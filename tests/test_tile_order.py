"""CPU check of the GEMM's XCD-aware workgroup -> tile map.

The kernel computes its output tile with ``jf::tile_of``
(``int8_block_quantized_amd/csrc/jf_tile_order.h``).  A skipped or duplicated
tile would leave part of the output unwritten or written twice; this test
compiles the same header for the host and checks on every grid up to 160 x 160
tiles that the map is a bijection.  (The GPU tests compare full outputs of the
grids the library actually launches.)
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_tile_map_is_a_bijection(tmp_path):
    exe = tmp_path / "tile_order_check"
    subprocess.run(["g++", "-O2", "-std=c++17", os.path.join(HERE, "tile_order_check.cpp"), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.split() == ["ok", str(160 * 160)]
