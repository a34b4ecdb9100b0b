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


def gemm_tolerance_check(gpu_bits, ref, K, absmag=None, label="", excl=None, rms=None):
    """|gpu - ref| <= 8e-3 |ref| + 1e-3 sqrt(K) rms(ref) on the checked entries.

    Entries whose term magnitudes sum to 2^127 or more (fp32 or BF16 overflow
    possible) are excluded from the tolerance and from rms; there the GPU value
    must be non-finite or within the tolerance.  They are given as term
    magnitudes (absmag) or directly as a boolean mask (excl).  rms, when given,
    is the rms of the checked entries of the whole output (for a check done
    panel by panel).  Returns the number excluded.
    """
    gpu = bf16_to_f64(gpu_bits)
    ref = np.asarray(ref, dtype=np.float64)
    if excl is None:
        excl = np.zeros(ref.shape, dtype=bool) if absmag is None else (absmag >= 2.0 ** 127)
    chk = ~excl
    if rms is None:
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


def whole_output_rms(ref, excl=None, panel=2048):
    """rms of the checked entries of a whole output, summed panel by panel."""
    ssum, cnt = 0.0, 0
    for r0 in range(0, ref.shape[0], panel):
        rp = ref[r0:r0 + panel]
        if excl is not None:
            rp = rp[~excl[r0:r0 + panel]]
        ssum += float(np.sum(rp * rp))
        cnt += rp.size
    return np.sqrt(ssum / cnt) if cnt else 0.0


def gemm_full_check(gpu_bits, ref, K, excl=None, label="", panel=2048):
    """Every entry of a (large) output against the tolerance, with rms taken
    over all checked entries of the whole output; the comparison runs in row
    panels to bound host memory.  Returns the number of excluded entries."""
    assert gpu_bits.shape == ref.shape, (gpu_bits.shape, ref.shape)
    rms = whole_output_rms(ref, excl, panel)
    n = 0
    for r0 in range(0, ref.shape[0], panel):
        n += gemm_tolerance_check(gpu_bits[r0:r0 + panel], ref[r0:r0 + panel], K, label=label,
                                  excl=None if excl is None else excl[r0:r0 + panel], rms=rms)
    return n


def overflow_candidate_rows(sa, sb, K):
    """Rows of A whose term magnitudes could sum to 2^127 or more, from the
    scale bytes alone: every |dq| is at most 448 * 2^(byte - 127), so a row's
    sum is at most K * 448^2 * 2^(max row byte + max byte of B - 254).  Rows
    under 2^127 by that bound cannot overflow."""
    a_max = np.max(sa, axis=1).astype(np.float64) if sa.shape[1] else np.zeros(sa.shape[0])
    b_max = float(np.max(sb)) if sb.size else 0.0
    log2_bound = np.log2(K * 448.0 * 448.0) + a_max + b_max - 254.0
    return np.nonzero(log2_bound >= 127.0)[0]
