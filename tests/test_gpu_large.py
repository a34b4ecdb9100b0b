"""Tensors beyond 2^32 elements or bytes: the quantizer's row+col+dbias launch with
packed scales on a [69632 x 65536] BF16 tensor (4.56 G elements, 9.1 GB), the
GEMM reading its rowwise codes as an A operand of 4.56 GB (K = 65536), and
the two rowwise-only quantize kernels on the same tensor.
Element offsets above 2^32 must be formed in 64 bits everywhere.

The tensor repeats one seeded 4096 x 4096 tile of the input generators (the
repetition is done by torch on the device), so every row and column of it is
known on the host: sampled rows and columns on both sides of element 2^32 are
compared with the oracle bit for bit, dbias within its summation bound, and
sampled GEMM rows within the GEMM tolerance."""

import numpy as np
import pytest

import mxfp8_block_scaled_quantize_amd as mx
import oracle
import workloads
from gpu_util import bf16_to_f64, gemm_tolerance_check, log, need_gpu, to_dev_bf16, to_host
from test_gpu_quantize import dbias_depth
from test_gpu_quantize_ex import unpack_words

pytestmark = pytest.mark.gpu

T = 4096
R, C = 69632, 65536          # R * C = 4.56e9 > 2^32; row 65536 starts at element 2^32


def test_quantize_and_gemm_beyond_2_pow_32_elements():
    torch = need_gpu()
    free, _ = torch.cuda.mem_get_info()
    if free < 40 * 2 ** 30:
        pytest.skip("needs about 24 GB of device memory (40 GB free asked for)")
    tile = workloads.normal_bf16((T, T), 77)
    log("large quantize R=%d C=%d (%.2e elements)" % (R, C, float(R) * C))
    x = to_dev_bf16(tile).repeat(R // T, C // T)
    assert x.shape == (R, C)
    out = mx.quantize(x, rowwise=True, colwise=True, dbias=True, packed=True)
    torch.cuda.synchronize()
    rows = [0, 4095, 65535, 65536, 65537, R - 1]
    for r in rows:
        q, s = oracle.quantize_rowwise(np.tile(tile[r % T], C // T)[None, :])
        assert np.array_equal(to_host(out["q_row"][r]), q[0]), r
        got_s = unpack_words(to_host(out["p_row"][:, r:r + 1]), 1)
        assert np.array_equal(got_s, s), r
    cols = [0, 4097, C // 2 + 31, C - 1]
    for c in cols:
        qT, sT = oracle.quantize_colwise(np.tile(tile[:, c % T], R // T)[:, None])
        assert np.array_equal(to_host(out["q_colT"][c]), qT[0]), c
        got_s = unpack_words(to_host(out["p_colT"][:, c:c + 1]), 1)
        assert np.array_equal(got_s, sT), c
    # dbias: R / T copies of each tile column sum, within the kernel's summation bound
    ref = (R // T) * oracle.dbias(tile).astype(np.float64)
    ref = np.tile(ref, C // T)
    mag = np.tile((R // T) * np.abs(bf16_to_f64(tile)).sum(axis=0), C // T)
    tol = 1.01 * dbias_depth(R) * 2.0 ** -24 * mag + np.abs(ref) * 2.0 ** -23 + 2.0 ** -126
    err = np.abs(to_host(out["dbias"]).astype(np.float64) - ref)
    assert np.all(err <= tol), "dbias off by %g" % (err - tol).max()
    # the GEMM with that rowwise copy as A (M = 69632, K = 65536: 4.56 GB of codes)
    N = 256
    b = workloads.normal_bf16((N, C), 78, std=0.02)
    qb = mx.quantize(to_dev_bf16(b), rowwise=True, packed=True)
    log("large gemm M=%d N=%d K=%d" % (R, N, C))
    y = mx.gemm(out["q_row"], out["p_row"], qb["q_row"], qb["p_row"])
    torch.cuda.synchronize()
    oqb, osb = oracle.quantize_rowwise(b)
    for r in rows:
        oqa, osa = oracle.quantize_rowwise(np.tile(tile[r % T], C // T)[None, :])
        ref = oracle.gemm_tn(oqa, osa, oqb, osb)
        gemm_tolerance_check(to_host(y[r:r + 1]), ref, C, label="row %d" % r)
    del out, y
    # the two rowwise-only kernels: the flat stream (byte scales) and the
    # panel kernel (packed scale words)
    for packed in (False, True):
        log("large rowwise quantize packed=%d" % packed)
        o = mx.quantize(x, rowwise=True, packed=packed)
        torch.cuda.synchronize()
        for r in rows:
            q, s = oracle.quantize_rowwise(np.tile(tile[r % T], C // T)[None, :])
            assert np.array_equal(to_host(o["q_row"][r]), q[0]), (packed, r)
            got_s = unpack_words(to_host(o["p_row"][:, r:r + 1]), 1) if packed else to_host(o["s_row"][r:r + 1])
            assert np.array_equal(got_s, s), (packed, r)
        del o


def test_grouped_gemm_with_experts_past_2_pow_32_bytes():
    """64 experts of 8192 x 8192 codes (4.3 GB of B: the last experts start
    past byte 2^32), 256 rows each: sampled rows of several experts, the last
    included, against the oracle with that expert's weights (every expert's
    weights differ: expert g's row j is row (j + 61 g) mod 4096 of the tile,
    repeated along K)."""
    torch = need_gpu()
    free, _ = torch.cuda.mem_get_info()
    if free < 40 * 2 ** 30:
        pytest.skip("needs about 14 GB of device memory (40 GB free asked for)")
    G, N, K, per = 64, 8192, 8192, 256
    M = G * per
    tile = workloads.normal_bf16((T, T), 79, std=0.02)
    base = to_dev_bf16(tile).repeat(N // T, K // T)                    # [8192, 8192]
    w = torch.stack([torch.roll(base, shifts=-61 * g, dims=0) for g in range(G)])   # [64, 8192, 8192]
    del base
    log("large grouped gemm G=%d N=%d K=%d" % (G, N, K))
    wq = mx.quantize(w.view(G * N, K), rowwise=True, packed=True)
    del w
    x = workloads.normal_bf16((M, K), 80)
    xq = mx.quantize(to_dev_bf16(x), rowwise=True, packed=True)
    off = torch.arange(0, M + 1, per, dtype=torch.int32, device="cuda")
    y = mx.grouped_gemm(xq["q_row"], xq["p_row"], wq["q_row"].view(G, N, K), wq["p_row"], off)
    torch.cuda.synchronize()
    cols = np.arange(0, N, 97)
    for g in (0, 31, 62, 63):
        wg = np.tile(tile[(np.arange(N) + 61 * g) % T][cols], (1, K // T))     # the sampled weight rows
        oqw, osw = oracle.quantize_rowwise(wg)
        for r in (g * per, g * per + per - 1):
            oqx, osx = oracle.quantize_rowwise(x[r:r + 1])
            ref = oracle.gemm_tn(oqx, osx, oqw, osw)
            gemm_tolerance_check(to_host(y[r:r + 1])[:, cols], ref, K, label="expert %d row %d" % (g, r))


def test_gemm_output_past_2_pow_32_elements():
    """C [69632 x 65536] (4.56 G outputs, 9.1 GB of BF16) with K = 128, and the
    same GEMM writing MXFP8 (4.56 GB of codes): sampled rows on both sides of
    element 2^32 against the oracle's product; the MXFP8 rows must equal the
    library's rowwise quantization of the BF16 rows of the first launch (the
    output quantizer's contract: a consistency check between entry points)."""
    torch = need_gpu()
    free, _ = torch.cuda.mem_get_info()
    if free < 40 * 2 ** 30:
        pytest.skip("needs about 15 GB of device memory (40 GB free asked for)")
    M, N, K = R, C, 128
    a = workloads.normal_bf16((M, K), 81)
    b = workloads.normal_bf16((N, K), 82, std=0.25)
    qa = mx.quantize(to_dev_bf16(a), rowwise=True, packed=True)
    qb = mx.quantize(to_dev_bf16(b), rowwise=True, packed=True)
    log("large gemm output M=%d N=%d K=%d" % (M, N, K))
    y = mx.gemm(qa["q_row"], qa["p_row"], qb["q_row"], qb["p_row"])
    torch.cuda.synchronize()
    oqb, osb = oracle.quantize_rowwise(b)
    rows = [0, 65535, 65536, M - 1]
    want = {}
    for r in rows:
        oqa, osa = oracle.quantize_rowwise(a[r:r + 1])
        gemm_tolerance_check(to_host(y[r:r + 1]), oracle.gemm_tn(oqa, osa, oqb, osb), K, label="row %d" % r)
        rq = mx.quantize(y[r:r + 1].contiguous(), rowwise=True, packed=True)   # the quantizer on the BF16 row
        want[r] = (to_host(rq["q_row"]), to_host(rq["p_row"]))
    del y
    q, p = mx.gemm(qa["q_row"], qa["p_row"], qb["q_row"], qb["p_row"], mxfp8_out=True)
    torch.cuda.synchronize()
    for r in rows:
        assert np.array_equal(to_host(q[r:r + 1]), want[r][0]), r
        assert np.array_equal(to_host(p[:, r:r + 1]), want[r][1]), r
