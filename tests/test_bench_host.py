"""bench.py host logic (CPU): the HBM traffic it reports for the dominant
GEMM family comes from the committed rocprofv3 counter summary only while
that summary was taken on the current GEMM sources."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FAMILIES = [f"gemm_i8bs tA={a} tB={b} i8-out" for a, b in ((0, 0), (0, 1), (1, 0))]


def test_summary_lists_every_family_with_plausible_bytes():
    tr = bench.read_traffic()
    assert tr is not None and "source_digest" in tr
    for fam in FAMILIES:
        v = int(tr[f"traffic[{fam}]"])
        # the hidden-4096 GEMMs move at least their operands, output and scales
        # once (0.19-0.24 GB per launch) and, with L2 re-reads, well under 10x that
        assert 1.5e8 < v < 2.5e9, (fam, v)


def test_traffic_used_only_for_the_sources_it_was_taken_on(monkeypatch):
    tr = bench.read_traffic()
    monkeypatch.setattr(bench, "source_digest", lambda: tr["source_digest"])
    for fam in FAMILIES:
        assert bench.profile_traffic(fam) == int(tr[f"traffic[{fam}]"])
    assert bench.profile_traffic("gelu_i8") is None
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 16)
    for fam in FAMILIES:
        assert bench.profile_traffic(fam) is None


def test_source_digest_covers_the_gemm_sources(tmp_path, monkeypatch):
    """Changing any of the files the digest covers changes the digest."""
    pkg = tmp_path / "int8_block_quantized_amd"
    (pkg / "csrc").mkdir(parents=True)
    files = ("csrc/gemm.hip", "csrc/jf_tile_order.h", "csrc/jf_device.h", "_build.py")
    for f in files:
        (pkg / f).write_bytes(open(os.path.join(ROOT, "int8_block_quantized_amd", f), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.source_digest()
    assert d0 == bench.source_digest()
    for f in files:
        p = pkg / f
        orig = p.read_bytes()
        p.write_bytes(orig + b"\n")
        assert bench.source_digest() != d0, f
        p.write_bytes(orig)
    assert bench.source_digest() == d0
