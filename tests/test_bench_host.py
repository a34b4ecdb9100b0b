"""Host-side checks of bench.py that need no GPU: the one-GPU guard, the
algorithmic byte count, and that the committed rocprofv3 summaries carry
traffic lines for the current GEMM sources for every workload's dominant
GEMM."""

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


def test_profiles_match_the_gemm_sources():
    """Each workload's dominant GEMM has a traffic line taken on the current GEMM sources."""
    for key in ("gemm:8192x14336x4096", "gemm:4096x4096x16384", "gemm:grouped:16384x14336x4096:G=8",
                "gemm:32768x8192x8192", "gemm:fprop:8192x14336x4096", "gemm:fc1:8192x14336x4096",
                "gemm:grouped:relu^2:16384x14336x4096:G=8"):
        got = bench.profiled_traffic(key)
        assert got is not None, key
        nbytes, fname = got
        assert nbytes > 0 and os.path.exists(os.path.join(ROOT, "profiles", fname))


def test_profiles_match_the_quantize_sources():
    """The largest quantize launch of each workload has a traffic line taken
    on the current quantizer sources (reported as quantize_roofline.traffic)."""
    for key in ("quantize:A[8192x8192]:packed", "quantize:dY[16384x4096]:row+col+dbias:packed",
                "quantize:W[8x14336x4096]", "quantize:W[8x14336x4096]:packed",
                "quantize:A[32768x8192]:row+col:packed", "quantize:dY[8192x14336]:row+col:packed",
                "quantize:dH=dA*2relu(H)[8192x14336]:row+col+dbias:packed"):
        got = bench.profiled_traffic(key, bench.QUANTIZE_SOURCES)
        assert got is not None, key
        assert got[0] > 0


def test_profiles_are_short_text():
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        assert name.endswith((".md", ".txt")), name
        assert os.path.getsize(os.path.join(ROOT, "profiles", name)) < 64 * 1024, name
