"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

import os
import sys

import numpy as np
import pytest

import mxfp8_block_scaled_quantize_amd as mx
from mxfp8_block_scaled_quantize_amd import build as mxbuild


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(mx.LIB_PATH):
        mxbuild.build()
    mx.lib()
    return torch


def log(msg):
    sys.stdout.write("[case] %s\n" % msg)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.cpu().numpy().view(np.uint32)
    return t.cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_tolerance_check(gpu_bits, ref, K, absmag=None, label=""):
    """|gpu - ref| <= 8e-3 |ref| + 1e-3 sqrt(K) rms(ref) on the checked entries.

    Entries whose term magnitudes sum to 2^127 or more (fp32 or BF16 overflow
    possible) are excluded from the tolerance and from rms; there the GPU value
    must be non-finite or within the tolerance.  Returns the number excluded.
    """
    gpu = bf16_to_f64(gpu_bits)
    ref = np.asarray(ref, dtype=np.float64)
    excl = np.zeros(ref.shape, dtype=bool) if absmag is None else (absmag >= 2.0 ** 127)
    chk = ~excl
    rms = np.sqrt(np.mean(ref[chk] ** 2)) if chk.any() else 0.0
    tol = 8e-3 * np.abs(ref) + 1e-3 * np.sqrt(K) * rms
    err = np.abs(gpu - ref)
    bad = chk & ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:8]
        detail = ", ".join("(%d,%d) gpu=%g ref=%g tol=%g" % (i, j, gpu[i, j], ref[i, j], tol[i, j]) for i, j in idx)
        raise AssertionError("%s: %d of %d entries out of tolerance: %s" % (label, bad.sum(), chk.sum(), detail))
    if excl.any():
        ok = ~np.isfinite(gpu[excl]) | (err[excl] <= tol[excl])
        assert ok.all(), "%s: overflow-excluded entries neither non-finite nor in tolerance" % label
    return int(excl.sum())


def sample_indices(n, count, seed, tile=128):
    """Sorted sample of row/column indices including both ends and tile edges."""
    rng = np.random.default_rng(seed)
    fixed = {0, 1, n - 1, n - 2}
    for t in (tile, 2 * tile, n // 2):
        for d in (-1, 0, 1):
            if 0 <= t + d < n:
                fixed.add(t + d)
    rest = rng.choice(n, size=min(count, n), replace=False)
    return np.array(sorted(fixed | set(int(v) for v in rest)), dtype=np.int64)
