"""Host-side checks of bench.py that need no GPU: the one-GPU guard, the
algorithmic byte count, the keying of profile traffic to the kernel sources,
and the form of the committed rocprofv3 summaries."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_quant_bytes():
    # read 2 B per element and input, write 1 + 1/32 B per element and copy, 4 B per column of dbias
    assert bench.quant_bytes(32, 64, 1) == 32 * 64 * (2 + 33 / 32)
    assert bench.quant_bytes(32, 64, 2, dbias=True) == 32 * 64 * (2 + 2 * 33 / 32) + 4 * 64
    assert bench.quant_bytes(32, 64, 2, inputs=2) == 32 * 64 * (4 + 2 * 33 / 32)


def test_profiled_traffic_is_keyed_to_the_kernel_sources(tmp_path, monkeypatch):
    """A profile's traffic line counts only while the kernel's sources hash to
    the value it was taken on: the same line under another hash is ignored
    (the bench then reports traffic null)."""
    src = bench.source_hash(bench.GEMM_SOURCES)
    pdir = tmp_path / "profiles"
    pdir.mkdir()
    (pdir / "a.md").write_text("traffic gemm:1x2x3 src=%s read_bytes=10 write_bytes=5\n"
                               "traffic gemm:4x5x6 src=0000000000000000 read_bytes=1 write_bytes=1\n" % src)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda files=bench.GEMM_SOURCES: src)
    assert bench.profiled_traffic("gemm:1x2x3") == (15, "a.md")
    assert bench.profiled_traffic("gemm:4x5x6") is None
    assert bench.profiled_traffic("gemm:7x8x9") is None


def test_profiles_are_well_formed():
    """Every committed summary gives the rocprofv3 commands that made it (run on
    committed files only) and its traffic lines name a kernel, a source hash
    and byte counts."""
    pdir = os.path.join(ROOT, "profiles")
    names = sorted(os.listdir(pdir))
    assert names
    for name in names:
        text = open(os.path.join(pdir, name)).read()
        assert "rocprofv3" in text, name
        assert "_work" not in text, name
        for line in text.splitlines():
            parts = line.split()
            if parts[:1] == ["traffic"]:
                assert len(parts) == 5 and parts[2].startswith("src=") and len(parts[2]) == 20, (name, line)
                kv = dict(p.split("=", 1) for p in parts[3:])
                assert int(kv["read_bytes"]) > 0 and int(kv["write_bytes"]) > 0, (name, line)


def test_profiles_are_short_text():
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        assert name.endswith((".md", ".txt")), name
        assert os.path.getsize(os.path.join(ROOT, "profiles", name)) < 64 * 1024, name
