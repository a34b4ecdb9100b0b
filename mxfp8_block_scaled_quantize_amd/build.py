"""Build libmxfp8.so (gfx950 HIP kernels + C ABI) in-tree with hipcc, and
libmxfp8_calib.so, the benchmark's measurement aid (the register-only MFMA
rate; not part of the library)."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libmxfp8.so")
CALIB_PATH = os.path.join(HERE, "libmxfp8_calib.so")
SOURCES = ["api.hip", "quantize.hip", "pack_scales.hip", "gemm.hip"]
CALIB_SOURCES = ["calib.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 VALU forms are disabled for all device code; hipcc's host pass
# warns that it does not know the feature, which is harmless.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option"]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES + CALIB_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = False
    for cmd, p in procs:
        out, _ = p.communicate()
        text = "\n".join(line for line in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in line)
        if p.returncode != 0:
            failed = True
            sys.stderr.write("FAILED: %s\n%s\n" % (" ".join(cmd), text))
        elif verbose and text.strip():
            sys.stderr.write(text + "\n")
    if failed:
        raise RuntimeError("hipcc compilation failed")
    n = len(SOURCES)
    for path, parts in ((LIB_PATH, objs[:n]), (CALIB_PATH, objs[n:])):
        tmp = path + ".tmp%d" % os.getpid()
        subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *parts, "-o", tmp])
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
