"""GPU parity of mxfp8_pack_scales (bit-exact), mxfp8_gemm and
mxfp8_grouped_gemm against the CPU oracle (BF16 outputs within
|gpu - ref| <= 8e-3 |ref| + 1e-3 sqrt(K) rms(ref); exact where the exact
result is a BF16 value)."""

import numpy as np
import pytest

import mxfp8_block_scaled_quantize_amd as mx
import oracle
import workloads
from gpu_util import (bf16_to_f64, gemm_full_check, gemm_tolerance_check, log, need_gpu,
                      overflow_candidate_rows, to_dev, to_dev_bf16, to_host, whole_output_rms)

pytestmark = pytest.mark.gpu


def quantize_on_gpu(bits, colwise=False):
    """Rowwise (or transposed columnwise) MXFP8 copy made by the GPU path,
    with its packed scales; all device tensors."""
    need_gpu()
    x = to_dev_bf16(bits)
    out = mx.quantize(x, rowwise=not colwise, colwise=colwise)
    q, s = (out["q_colT"], out["s_colT"]) if colwise else (out["q_row"], out["s_row"])
    return q, s, mx.pack_scales(s)


def gemm_gpu(qa, pa, qb, pb, ldc=None, canary=False, flags=0):
    torch = need_gpu()
    M, K = qa.shape
    N = qb.shape[0] // (2 if flags & mx.MXFP8_GEMM_SWIGLU else 1)   # SwiGLU: B holds gate and up rows
    ldc = N if ldc is None else ldc
    G = 1024 if canary else 0
    full = torch.full((M * ldc + 2 * G,), -12345, dtype=torch.int16, device="cuda")
    c = full[G:G + M * ldc].view(torch.bfloat16)
    mx.mxfp8_gemm_ex(qa, pa, qb, pb, c, ldc, M, N, K, flags)
    torch.cuda.synchronize()
    h = to_host(full.view(torch.bfloat16))
    if canary:
        assert np.all(h[:G] == np.uint16(-12345 & 0xFFFF)) and np.all(h[-G:] == np.uint16(-12345 & 0xFFFF))
        inner = h[G:G + M * ldc].reshape(M, ldc)
        assert np.all(inner[:, N:] == np.uint16(-12345 & 0xFFFF)), "columns beyond N written"
    return h[G:G + M * ldc].reshape(M, ldc)[:, :N]


# ------------------------------------------------------------- packing

@pytest.mark.parametrize("dim,K", [(32, 128), (96, 512), (1000, 4096), (64, 128 * 67), (264, 2560), (1004, 1024),
                                   (16384, 4096)])
def test_pack_scales_bit_exact(dim, K):
    """Both kernel forms: 4-byte accesses (K / 128 or dim not a multiple of 4,
    or a source stride not a multiple of 16) and 16-byte accesses (partial row
    and word tiles included)."""
    torch = need_gpu()
    rng = np.random.default_rng(dim + K)
    s = rng.integers(0, 256, size=(dim, K // 32)).astype(np.uint8)
    log("pack dim=%d K=%d" % (dim, K))
    got = to_host(mx.pack_scales(to_dev(s)))
    assert np.array_equal(got, oracle.pack_scales(s))
    # strided sources (ld_s > K/32; + 12 keeps the 4-byte form, + 16 allows the 16-byte one)
    for extra in (12, 16):
        wide = np.zeros((dim, K // 32 + extra), dtype=np.uint8)
        wide[:, :K // 32] = s
        ws = to_dev(wide)
        out = torch.empty((K // 128, dim), dtype=torch.int32, device="cuda")
        mx.mxfp8_pack_scales(ws, dim, K, wide.shape[1], out)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(out), oracle.pack_scales(s)), extra


# -------------------------------------------------------- dense GEMM

def check_dense(a_bits, b_bits, label, rows=None, cols=None, ldc=None, canary=False):
    qa, sa, pa = quantize_on_gpu(a_bits)
    qb, sb, pb = quantize_on_gpu(b_bits)
    K = a_bits.shape[1]
    log("%s M=%d N=%d K=%d" % (label, a_bits.shape[0], b_bits.shape[0], K))
    c = gemm_gpu(qa, pa, qb, pb, ldc=ldc, canary=canary)
    # oracle on its own quantization of the same inputs
    oqa, osa = oracle.quantize_rowwise(a_bits)
    oqb, osb = oracle.quantize_rowwise(b_bits)
    ref = oracle.gemm_tn(oqa, osa, oqb, osb, rows=rows, cols=cols)
    mag = oracle.gemm_tn_abs(oqa, osa, oqb, osb, rows=rows, cols=cols)
    sub = c if rows is None else c[np.ix_(rows, cols)]
    return gemm_tolerance_check(sub, ref, K, mag, label), sub, ref


def test_tiny_config():
    d = workloads.tiny()
    check_dense(d["A"], d["B"], "tiny", canary=True)


@pytest.mark.parametrize("M,N,K", [(32, 32, 128), (96, 224, 384), (160, 96, 1024), (1000, 320, 256),
                                   (7, 64, 128), (256, 4096, 128), (130, 160, 2048), (288, 288, 1152),
                                   # 10 x 3 and 3 x 11 tiles of 256: the L2 groups of 4 tiles along the
                                   # larger dimension end in a partial group, and the tile count is not
                                   # a multiple of the 8 XCDs (both branches of the tile remap)
                                   (2520, 736, 256), (700, 2784, 256)])
def test_ragged_gemm_shapes(M, N, K):
    a = workloads.normal_bf16((M, K), M + K)
    b = workloads.normal_bf16((N, K), N + 3 * K, std=0.5)
    check_dense(a, b, "ragged", ldc=N + 24, canary=True)


def test_identity_gives_dequantized_b_exactly():
    a = (np.eye(256, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    b = workloads.normal_bf16((256, 256), 1)
    qa, sa, pa = quantize_on_gpu(a)
    qb, sb, pb = quantize_on_gpu(b)
    log("identity")
    c = gemm_gpu(qa, pa, qb, pb)
    want = oracle.dequantize(*oracle.quantize_rowwise(b)).T
    assert np.array_equal(bf16_to_f64(c), want)


def test_small_integers_exact():
    rng = np.random.default_rng(10)
    A = rng.integers(-14, 15, size=(192, 640))
    B = rng.integers(-14, 15, size=(160, 640))
    ab = (A.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bb = (B.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    qa, sa, pa = quantize_on_gpu(ab)
    qb, sb, pb = quantize_on_gpu(bb)
    log("integers")
    c = gemm_gpu(qa, pa, qb, pb)
    exact = (A @ B.T).astype(np.float64)
    # every |sum| < 2^16 here; BF16 keeps 8 significant bits: compare against
    # the round-to-nearest-even BF16 of the exact integer
    want = bf16_to_f64(workloads.f32_to_bf16_bits(exact.astype(np.float32)))
    assert np.array_equal(bf16_to_f64(c), want)


def test_one_scale_byte_doubles_exactly_its_block():
    # P8: bump one E8M0 byte of A (row 37, K-block 5) by one: only row 37
    # changes, and only through K [160, 192).  A tile spanning several MFMA
    # blocks (256 x 256 x 512) catches scale-layout mistakes.
    torch = need_gpu()
    a = workloads.normal_bf16((256, 512), 21)
    b = workloads.normal_bf16((256, 512), 22)
    qa, sa, pa = quantize_on_gpu(a)
    qb, sb, pb = quantize_on_gpu(b)
    base = gemm_gpu(qa, pa, qb, pb)
    sa2 = sa.clone()
    sa2[37, 5] += 1
    pa2 = mx.pack_scales(sa2)
    log("one-hot scale")
    c2 = gemm_gpu(qa, pa2, qb, pb)
    assert np.array_equal(np.delete(c2, 37, 0), np.delete(base, 37, 0))
    oqa, osa = oracle.quantize_rowwise(a)
    oqb, osb = oracle.quantize_rowwise(b)
    osa2 = osa.copy()
    osa2[37, 5] += 1
    ref = oracle.gemm_tn(oqa, osa2, oqb, osb, rows=[37])
    gemm_tolerance_check(c2[37:38], ref, 512, label="bumped row")
    delta = oracle.gemm_tn(oqa[:, 160:192], osa[:, 5:6], oqb[:, 160:192], osb[:, 5:6], rows=[37])
    assert np.abs(delta).max() > 0
    _ = torch


@pytest.mark.slow
def test_largest_k():
    """K = 2^22, the largest K the library accepts (a 256-row operand tile is
    then 2^30 bytes of buffer range), with a ragged second row tile
    (M = 288): random E4M3 codes (NaN patterns excluded) and scale bytes
    120..127 made on the device, the sampled entries checked against the
    oracle on the same codes."""
    torch = need_gpu()
    M, N, K = 288, 256, 1 << 22
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)

    def codes(rows):
        c = torch.randint(0, 254, (rows, K), dtype=torch.uint8, device="cuda", generator=gen)
        return torch.where(c >= 0x7F, c + 1, c)

    qa, qb = codes(M), codes(N)
    sa = torch.randint(120, 128, (M, K // 32), dtype=torch.uint8, device="cuda", generator=gen)
    sb = torch.randint(120, 128, (N, K // 32), dtype=torch.uint8, device="cuda", generator=gen)
    log("largest K: M=%d N=%d K=%d" % (M, N, K))
    c = gemm_gpu(qa, mx.pack_scales(sa), qb, mx.pack_scales(sb))
    rows = np.array([0, 1, 100, 255, 256, 270, 287])
    cols = np.array([0, 31, 128, 200, 255])
    ref = oracle.gemm_tn(qa[rows].cpu().numpy(), sa[rows].cpu().numpy(), qb[cols].cpu().numpy(),
                         sb[cols].cpu().numpy())
    gemm_tolerance_check(c[np.ix_(rows, cols)], ref, K, label="K=2^22")


@pytest.mark.parametrize("flags", [0, mx.MXFP8_GEMM_SQRELU, mx.MXFP8_GEMM_GELU, mx.MXFP8_GEMM_SWIGLU])
def test_k_zero_writes_zeros(flags):
    """K = 0: the product is 0, and so are relu(0)^2, GELU(0) and SiLU(0) * 0;
    the dense and the grouped entry points write +0 everywhere they own."""
    torch = need_gpu()
    c = torch.full((64, 96), 3.0, dtype=torch.bfloat16, device="cuda")
    mx.mxfp8_gemm_ex(None, None, None, None, c, 96, 64, 96, 0, flags)
    torch.cuda.synchronize()
    assert torch.all(c.view(torch.int16) == 0).item()
    g = torch.full((64, 96), 3.0, dtype=torch.bfloat16, device="cuda")
    off = to_dev(np.array([0, 20, 20, 50], dtype=np.int32))
    mx.mxfp8_grouped_gemm_ex(None, None, None, None, off, 3, g, 96, 64, 96, 0, flags)
    torch.cuda.synchronize()
    gh = to_host(g)
    assert np.all(gh[:50] == 0) and np.all(bf16_to_f64(gh[50:]) == 3.0)


# ------------------------------------------------ accumulate (beta = 1)

@pytest.mark.parametrize("M,N,K", [(96, 224, 384), (300, 288, 1152), (512, 512, 2048)])
def test_gemm_accumulate(M, N, K):
    """C = C_old + A B^T, rounded once: compared with the oracle product plus the
    old values; columns beyond N (ldc padding) keep their canary."""
    torch = need_gpu()
    a = workloads.normal_bf16((M, K), M + 7 * K)
    b = workloads.normal_bf16((N, K), N + 11 * K, std=0.05)
    c_old = workloads.normal_bf16((M, N), M * N + 1, std=4.0)
    qa, sa, pa = quantize_on_gpu(a)
    qb, sb, pb = quantize_on_gpu(b)
    ldc = N + 40
    full = np.full((M, ldc), 0x3F80, dtype=np.uint16)        # 1.0 in the padding
    full[:, :N] = c_old
    cd = to_dev_bf16(full)
    log("accumulate M=%d N=%d K=%d" % (M, N, K))
    mx.mxfp8_gemm_ex(qa, pa, qb, pb, cd, ldc, M, N, K, mx.MXFP8_GEMM_ACCUMULATE)
    torch.cuda.synchronize()
    got = to_host(cd)
    assert np.all(got[:, N:] == 0x3F80), "ldc padding written"
    oqa, osa = oracle.quantize_rowwise(a)
    oqb, osb = oracle.quantize_rowwise(b)
    ref = oracle.gemm_tn(oqa, osa, oqb, osb) + bf16_to_f64(c_old)
    gemm_tolerance_check(got[:, :N], ref, K, label="accumulate")


def test_gemm_accumulate_exact_on_integers():
    """Small integers: every partial sum is exact in fp32, so C_old + A B^T must be
    the exact integer rounded once to BF16."""
    torch = need_gpu()
    rng = np.random.default_rng(21)
    M, N, K = 128, 96, 256
    ai = rng.integers(-3, 4, size=(M, K)).astype(np.float32)
    bi = rng.integers(-3, 4, size=(N, K)).astype(np.float32)
    ci = rng.integers(-40, 41, size=(M, N)).astype(np.float32)
    a = workloads.f32_to_bf16_bits(ai)
    b = workloads.f32_to_bf16_bits(bi)
    c_old = workloads.f32_to_bf16_bits(ci)
    qa, sa, pa = quantize_on_gpu(a)
    qb, sb, pb = quantize_on_gpu(b)
    cd = to_dev_bf16(c_old)
    mx.gemm(qa, pa, qb, pb, out=cd, accumulate=True)
    torch.cuda.synchronize()
    exact = ai.astype(np.int64) @ bi.astype(np.int64).T + ci.astype(np.int64)
    want = workloads.f32_to_bf16_bits(exact.astype(np.float32))
    assert np.array_equal(to_host(cd), want)


def test_gemm_accumulate_k_zero_keeps_c():
    torch = need_gpu()
    c_old = workloads.normal_bf16((64, 96), 5)
    cd = to_dev_bf16(c_old)
    mx.mxfp8_gemm_ex(None, None, None, None, cd, 96, 64, 96, 0, mx.MXFP8_GEMM_ACCUMULATE)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(cd), c_old)


# --------------------------------------------------------- grouped GEMM

def grouped_case(M, N, K, counts, seed, canary_rows=True, accumulate=False, sqrelu=False, gelu=False,
                 swiglu=False, bias=False):
    torch = need_gpu()
    G = len(counts)
    NB = 2 * N if swiglu else N   # SwiGLU: per expert N gate rows, then N up rows
    x = workloads.normal_bf16((M, K), seed)
    w = workloads.normal_bf16((G, NB, K), seed + 1, std=0.02)
    off = workloads.offsets_from_counts(counts)
    qx, sx, px = quantize_on_gpu(x)
    wq = quantize_on_gpu(w.reshape(G * NB, K))
    qw = wq[0].view(G, NB, K)
    pw = wq[2]
    c_old = workloads.normal_bf16((M, N), seed + 2, std=2.0) if accumulate else None
    if accumulate:
        out = to_dev_bf16(c_old)
    else:
        out = torch.full((M, N), -7.0, dtype=torch.bfloat16, device="cuda")
    log("grouped M=%d N=%d K=%d counts=%s accumulate=%d" % (M, N, K, list(counts), accumulate))
    bb = workloads.normal_bf16((G, NB), seed + 3, std=0.5) if bias else None   # one bias row per expert
    mx.grouped_gemm(qx, px, qw, pw, to_dev(off), out=out, accumulate=accumulate, sqrelu=sqrelu, gelu=gelu,
                    swiglu=swiglu, bias=None if bb is None else to_dev_bf16(bb))
    torch.cuda.synchronize()
    c = to_host(out)
    oqx, osx = oracle.quantize_rowwise(x)
    oq = [oracle.quantize_rowwise(w[g]) for g in range(G)]
    qwo = np.stack([q for q, _ in oq])
    swo = np.stack([s for _, s in oq])
    covered = np.zeros(M, dtype=bool)
    covered[off[0]:off[-1]] = True
    rows = np.nonzero(covered)[0]
    ref = oracle.grouped_gemm_tn(oqx, osx, qwo, swo, off, rows=rows)
    if accumulate:
        ref = ref + bf16_to_f64(c_old[rows])
    t = None
    if bias:
        t = product_bound(ref, K)
        grp = np.searchsorted(off, rows, side="right") - 1                  # expert of each covered row
        ref = ref + bf16_to_f64(bb)[grp]                                     # R + bias[g] (exact)
    if sqrelu:
        sqrelu_tolerance_check(c[rows], ref, K, label="grouped sqrelu", t=t)
    elif gelu:
        gelu_tolerance_check(c[rows], ref, K, label="grouped gelu", t=t)
    elif swiglu:
        swiglu_tolerance_check(c[rows], ref, K, label="grouped swiglu", t=t)
    elif bias:
        bias_tolerance_check(c[rows], ref, t, label="grouped bias")
    else:
        gemm_tolerance_check(c[rows], ref, K, label="grouped")
    if canary_rows and accumulate:
        assert np.array_equal(c[~covered], c_old[~covered]), "rows outside the groups were written"
    elif canary_rows:
        assert np.all(bf16_to_f64(c[~covered]) == -7.0), "rows outside the groups were written"


def sqrelu_tolerance_check(gpu_bits, r, K, label="", rms=None, t=None):
    """relu(R)^2 epilogue: the GPU forms relu(acc)^2 from its fp32 sum acc,
    |acc - R| <= t = 8e-3 |R| + 1e-3 sqrt(K) rms(R) (the GEMM bound), so
    |relu(acc)^2 - relu(R)^2| <= t (2|R| + t), plus the one BF16 rounding,
    2^-9 (|R| + t)^2 (doubled for margin)."""
    gpu = bf16_to_f64(gpu_bits)
    r = np.asarray(r, dtype=np.float64)
    if t is None:   # (a bias test passes the bound of the unbiased product)
        if rms is None:
            rms = np.sqrt(np.mean(r ** 2))
        t = 8e-3 * np.abs(r) + 1e-3 * np.sqrt(K) * rms
    tol = t * (2 * np.abs(r) + t) + 2.0 ** -8 * (np.abs(r) + t) ** 2
    err = np.abs(gpu - oracle.sqrelu_epilogue(r))
    bad = ~(err <= tol)
    assert not bad.any(), "%s: %d entries out of tolerance, worst %g vs %g" % (
        label, bad.sum(), err[bad].max(), tol[bad][np.argmax(err[bad])])
    assert np.all(gpu >= 0.0), label


@pytest.mark.parametrize("M,N,K", [(32, 32, 128), (160, 96, 1024), (1000, 320, 256), (288, 288, 1152)])
def test_gemm_sqrelu_epilogue(M, N, K):
    a = workloads.normal_bf16((M, K), 3 * M + K)
    b = workloads.normal_bf16((N, K), 5 * N + K, std=0.5)
    qa, sa, pa = quantize_on_gpu(a)
    qb, sb, pb = quantize_on_gpu(b)
    log("sqrelu epilogue M=%d N=%d K=%d" % (M, N, K))
    c = gemm_gpu(qa, pa, qb, pb, ldc=N + 24, canary=True, flags=mx.MXFP8_GEMM_SQRELU)
    oqa, osa = oracle.quantize_rowwise(a)
    oqb, osb = oracle.quantize_rowwise(b)
    sqrelu_tolerance_check(c, oracle.gemm_tn(oqa, osa, oqb, osb), K, "sqrelu")


def test_gemm_sqrelu_epilogue_exact_on_integers():
    """Integer operands: the fp32 sum is exact, its square is exact in fp32
    (< 2^24), so the output is the BF16 rounding of relu(R)^2 exactly."""
    rng = np.random.default_rng(12)
    A = rng.integers(-3, 4, size=(160, 256))
    B = rng.integers(-3, 4, size=(96, 256))
    ab = (A.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bb = (B.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    qa, sa, pa = quantize_on_gpu(ab)
    qb, sb, pb = quantize_on_gpu(bb)
    log("sqrelu integers")
    c = gemm_gpu(qa, pa, qb, pb, flags=mx.MXFP8_GEMM_SQRELU)
    v = oracle.sqrelu_epilogue((A @ B.T).astype(np.float64))
    assert v.max() < 2.0 ** 24
    want = bf16_to_f64(workloads.f32_to_bf16_bits(v.astype(np.float32)))
    assert np.array_equal(bf16_to_f64(c), want)


def test_grouped_sqrelu_epilogue():
    grouped_case(1200, 96, 256, [5, 0, 131, 257, 600], 9, sqrelu=True)


GELU_MIN = -0.16997   # min GELU, at x = -0.7518 (GELU(-0.75179) = -0.169971)


def gelu_tolerance_check(gpu_bits, r, K, label="", rms=None, t=None):
    """GELU(R) epilogue: the GPU applies GELU to its fp32 sum acc with
    |acc - R| <= t (the GEMM bound); |GELU'| <= 1.13 everywhere, so the exact
    GELU moves by at most 1.13 t; the fp32 GELU adds (8 + 3 acc^2) 2^-24 of
    its value, and the BF16 rounding 2^-9 (doubled for margin)."""
    gpu = bf16_to_f64(gpu_bits)
    r = np.asarray(r, dtype=np.float64)
    if t is None:
        if rms is None:
            rms = np.sqrt(np.mean(r ** 2))
        t = 8e-3 * np.abs(r) + 1e-3 * np.sqrt(K) * rms
    g = oracle.gelu_epilogue(r)
    mag = np.abs(g) + 1.13 * t
    tol = 1.13 * t + 2.0 ** -8 * mag + (8.0 + 3.0 * (np.abs(r) + t) ** 2) * 2.0 ** -24 * mag
    err = np.abs(gpu - g)
    bad = ~(err <= tol)
    assert not bad.any(), "%s: %d entries out of tolerance, worst %g vs %g" % (
        label, bad.sum(), err[bad].max(), tol[bad][np.argmax(err[bad])])
    assert np.all(gpu >= GELU_MIN * (1 + 2.0 ** -7)), label


@pytest.mark.parametrize("M,N,K", [(32, 32, 128), (160, 96, 1024), (1000, 320, 256), (288, 288, 1152)])
def test_gemm_gelu_epilogue(M, N, K):
    a = workloads.normal_bf16((M, K), 7 * M + K)
    b = workloads.normal_bf16((N, K), 11 * N + K, std=0.5)
    qa, sa, pa = quantize_on_gpu(a)
    qb, sb, pb = quantize_on_gpu(b)
    log("gelu epilogue M=%d N=%d K=%d" % (M, N, K))
    c = gemm_gpu(qa, pa, qb, pb, ldc=N + 24, canary=True, flags=mx.MXFP8_GEMM_GELU)
    oqa, osa = oracle.quantize_rowwise(a)
    oqb, osb = oracle.quantize_rowwise(b)
    gelu_tolerance_check(c, oracle.gemm_tn(oqa, osa, oqb, osb), K, "gelu")


def test_gemm_gelu_epilogue_on_integers():
    """Integer operands: the fp32 sum R is exact, so the output is the BF16
    rounding of the fp32 GELU(R): between the BF16 roundings of GELU(R) -+ its
    fp32 error bound, i.e. the correctly rounded value unless GELU(R) is within
    that bound of a rounding boundary.  Far negative sums (R < -12) give
    values below 1e-30."""
    rng = np.random.default_rng(14)
    A = rng.integers(-1, 2, size=(160, 128))
    B = rng.integers(-1, 2, size=(96, 128))
    ab = (A.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bb = (B.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    qa, sa, pa = quantize_on_gpu(ab)
    qb, sb, pb = quantize_on_gpu(bb)
    log("gelu integers")
    c = bf16_to_f64(gemm_gpu(qa, pa, qb, pb, flags=mx.MXFP8_GEMM_GELU))
    R = (A @ B.T).astype(np.float64)
    g = oracle.gelu_epilogue(R)
    e = (8.0 + 3.0 * R * R) * 2.0 ** -24 * np.abs(g)
    near = R >= -12
    lo = bf16_to_f64(workloads.f32_to_bf16_bits((g - e).astype(np.float32)))
    hi = bf16_to_f64(workloads.f32_to_bf16_bits((g + e).astype(np.float32)))
    ok = (c >= lo) & (c <= hi)
    assert ok[near].all(), "%d of %d outside the rounding bracket" % ((~ok[near]).sum(), near.sum())
    assert np.all(np.abs(c[~near]) <= 1e-30)
    assert near.mean() > 0.9 and (lo == hi)[near].mean() > 0.99   # nearly every entry decided exactly


def test_grouped_gelu_epilogue():
    grouped_case(1200, 96, 256, [5, 0, 131, 257, 600], 10, gelu=True)


def swiglu_tolerance_check(gpu_bits, r, K, label="", rms=None, t=None):
    """SwiGLU epilogue on a product r [.., 2N] = [gate | up]: the GPU forms
    SiLU(g) * u from fp32 sums g, u with |g - R_g| <= t_g, |u - R_u| <= t_u (the
    GEMM bound, rms over the whole 2N-wide product); |SiLU'| <= 1.1, so
    |SiLU(g) u - SiLU(R_g) R_u| <= 1.1 t_g (|R_u| + t_u) + |SiLU(R_g)| t_u;
    plus the fp32 SiLU and product, (16 + 2 |g|) 2^-24 of the result, and the
    BF16 rounding, 2^-9 (doubled for margin)."""
    gpu = bf16_to_f64(gpu_bits)
    r = np.asarray(r, dtype=np.float64)
    n = r.shape[1] // 2
    if t is None:
        if rms is None:
            rms = np.sqrt(np.mean(r ** 2))
        t = 8e-3 * np.abs(r) + 1e-3 * np.sqrt(K) * rms
    rg, ru, tg, tu = r[:, :n], r[:, n:], t[:, :n], t[:, n:]
    want = oracle.swiglu_epilogue(r)
    m = (np.abs(oracle.silu_f64(rg)) + 1.1 * tg) * (np.abs(ru) + tu)
    tol = 1.1 * tg * (np.abs(ru) + tu) + np.abs(oracle.silu_f64(rg)) * tu + 2.0 ** -8 * m \
        + (16.0 + 2.0 * (np.abs(rg) + tg)) * 2.0 ** -24 * m
    err = np.abs(gpu - want)
    bad = ~(err <= tol)
    assert not bad.any(), "%s: %d entries out of tolerance, worst %g vs %g" % (
        label, bad.sum(), err[bad].max(), tol[bad][np.argmax(err[bad])])


@pytest.mark.parametrize("M,N,K", [(32, 32, 128), (160, 96, 1024), (1000, 320, 256), (288, 288, 1152),
                                   (300, 160, 640), (513, 384, 384)])
def test_gemm_swiglu_epilogue(M, N, K):
    """B = [gate; up] with 2N rows, C [M, N]; N not a multiple of 128 leaves
    a partial 64-row segment (and empty ones) in the last tile."""
    a = workloads.normal_bf16((M, K), 13 * M + K)
    b = workloads.normal_bf16((2 * N, K), 17 * N + K, std=0.5)
    qa, sa, pa = quantize_on_gpu(a)
    qb, sb, pb = quantize_on_gpu(b)
    log("swiglu epilogue M=%d N=%d K=%d" % (M, N, K))
    c = gemm_gpu(qa, pa, qb, pb, ldc=N + 24, canary=True, flags=mx.MXFP8_GEMM_SWIGLU)
    oqa, osa = oracle.quantize_rowwise(a)
    oqb, osb = oracle.quantize_rowwise(b)
    swiglu_tolerance_check(c, oracle.gemm_tn(oqa, osa, oqb, osb), K, "swiglu")


def test_gemm_swiglu_epilogue_on_integers():
    """Integer operands: the fp32 sums are exact, so the output is the BF16
    rounding of the fp32 SiLU(R_g) R_u: between the BF16 roundings of the
    exact value -+ its fp32 error bound (16 + 2 |R_g|) 2^-24 of it, which
    coincide except on BF16 rounding ties.  Gate and up rows differ, so a swapped pair
    or a gate paired with the wrong up column fails."""
    rng = np.random.default_rng(15)
    A = rng.integers(-1, 2, size=(160, 128))
    B = rng.integers(-1, 2, size=(192, 128))     # N = 96: gate rows 0..95, up rows 96..191
    ab = (A.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bb = (B.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    qa, sa, pa = quantize_on_gpu(ab)
    qb, sb, pb = quantize_on_gpu(bb)
    log("swiglu integers")
    c = bf16_to_f64(gemm_gpu(qa, pa, qb, pb, canary=True, flags=mx.MXFP8_GEMM_SWIGLU))
    R = (A @ B.T).astype(np.float64)
    v = oracle.swiglu_epilogue(R)
    e = (16.0 + 2.0 * np.abs(R[:, :96])) * 2.0 ** -24 * np.abs(v)
    lo = bf16_to_f64(workloads.f32_to_bf16_bits((v - e).astype(np.float32)))
    hi = bf16_to_f64(workloads.f32_to_bf16_bits((v + e).astype(np.float32)))
    ok = (c >= lo) & (c <= hi)
    assert ok.all(), "%d of %d outside the rounding bracket" % ((~ok).sum(), ok.size)
    # open: integer products on a BF16 tie (SiLU(g) = g to fp32 precision for large g)
    assert (lo == hi).mean() > 0.9


def test_grouped_swiglu_epilogue():
    grouped_case(1200, 96, 256, [5, 0, 131, 257, 600], 11, swiglu=True)
    grouped_case(700, 160, 384, [300, 0, 64, 336], 12, swiglu=True)


# ------------------------------------------------------------ bias epilogue

def product_bound(r, K):
    """The GEMM bound t on an (unbiased) product r, rms over all of r."""
    r = np.asarray(r, dtype=np.float64)
    return 8e-3 * np.abs(r) + 1e-3 * np.sqrt(K) * np.sqrt(np.mean(r ** 2))


def bias_tolerance_check(gpu_bits, ref_b, t, label=""):
    """|gpu - (R + b)| <= t (the bound of R) + the BF16 rounding of the
    biased value, 2^-9 |R + b| (doubled for margin)."""
    err = np.abs(bf16_to_f64(gpu_bits) - ref_b)
    tol = t + 2.0 ** -8 * (np.abs(ref_b) + t)
    bad = ~(err <= tol)
    assert not bad.any(), "%s: %d entries out of tolerance, worst %g" % (label, bad.sum(), err[bad].max())


BIAS_EPI = {"plain": 0, "sqrelu": mx.MXFP8_GEMM_SQRELU, "gelu": mx.MXFP8_GEMM_GELU, "swiglu": mx.MXFP8_GEMM_SWIGLU}


def bias_case(M, N, K, epi, seed, ldc=None):
    """C = epi(A B^T + bias) with a BF16 bias per B row (2N values for SwiGLU:
    gate, then up) of the same size as the products, so some sums cancel;
    ldc padding and canaries around C."""
    torch = need_gpu()
    NB = 2 * N if epi == "swiglu" else N
    a = workloads.normal_bf16((M, K), seed)
    b = workloads.normal_bf16((NB, K), seed + 1, std=0.25)
    bias = workloads.normal_bf16((NB,), seed + 2, std=2.0)
    qa, sa, pa = quantize_on_gpu(a)
    qb, sb, pb = quantize_on_gpu(b)
    log("bias epilogue %s M=%d N=%d K=%d ldc=%s seed=%d" % (epi, M, N, K, ldc, seed))
    ldc = N + 16 if ldc is None else ldc
    G = 1024
    full = torch.full((M * ldc + 2 * G,), -12345, dtype=torch.int16, device="cuda")
    c = full[G:G + M * ldc].view(torch.bfloat16)
    mx.mxfp8_gemm_bias(qa, pa, qb, pb, to_dev_bf16(bias), c, ldc, M, N, K, BIAS_EPI[epi])
    torch.cuda.synchronize()
    h = to_host(full.view(torch.bfloat16))
    canary = np.uint16(-12345 & 0xFFFF)
    assert np.all(h[:G] == canary) and np.all(h[-G:] == canary)
    inner = h[G:G + M * ldc].reshape(M, ldc)
    assert np.all(inner[:, N:] == canary), "columns beyond N written"
    got = inner[:, :N]
    oqa, osa = oracle.quantize_rowwise(a)
    oqb, osb = oracle.quantize_rowwise(b)
    r = oracle.gemm_tn(oqa, osa, oqb, osb)
    t = product_bound(r, K)
    rb = oracle.bias_add(r, bias)
    if epi == "plain":
        bias_tolerance_check(got, rb, t, "bias")
    elif epi == "sqrelu":
        sqrelu_tolerance_check(got, rb, K, "bias sqrelu", t=t)
    elif epi == "gelu":
        gelu_tolerance_check(got, rb, K, "bias gelu", t=t)
    else:
        swiglu_tolerance_check(got, rb, K, "bias swiglu", t=t)


@pytest.mark.parametrize("epi", ["plain", "sqrelu", "gelu", "swiglu"])
@pytest.mark.parametrize("M,N,K", [(160, 96, 512), (300, 288, 256), (64, 32, 128)])
def test_gemm_bias_epilogue(M, N, K, epi):
    bias_case(M, N, K, epi, 19 * M + 23 * N + K)


def test_gemm_bias_exact_on_integers():
    """Integer operands and an integer bias: R + b is exact in fp32 and BF16
    (|R + b| < 256), so the output equals it exactly; a bias taken from the
    wrong column, row or half fails."""
    rng = np.random.default_rng(16)
    A = rng.integers(-1, 2, size=(96, 128))
    B = rng.integers(-1, 2, size=(64, 128))
    bias = rng.integers(-100, 101, size=64).astype(np.float32)
    to_bits = lambda v: (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    qa, sa, pa = quantize_on_gpu(to_bits(A))
    qb, sb, pb = quantize_on_gpu(to_bits(B))
    log("bias integers")
    torch = need_gpu()
    c = torch.empty((96, 64), dtype=torch.bfloat16, device="cuda")
    mx.mxfp8_gemm_bias(qa, pa, qb, pb, to_dev_bf16(to_bits(bias)), c, 64, 96, 64, 128, 0)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_f64(to_host(c)), (A @ B.T + bias[None, :]).astype(np.float64))


def test_grouped_bias_epilogue():
    grouped_case(1200, 96, 256, [5, 0, 131, 257, 600], 13, bias=True)
    grouped_case(700, 160, 384, [300, 0, 64, 336], 14, bias=True, swiglu=True)
    grouped_case(900, 128, 256, [400, 200, 300], 15, bias=True, gelu=True)


@pytest.mark.parametrize("epi", ["plain", "gelu", "swiglu"])
def test_bias_with_k_zero_writes_the_epilogue_of_the_bias(epi):
    """K = 0: C = epi(bias) on every row (SwiGLU: SiLU(gate bias) * up bias)."""
    torch = need_gpu()
    N = 96
    NB = 2 * N if epi == "swiglu" else N
    bias = workloads.normal_bf16((NB,), 33, std=2.0)
    c = torch.full((40, N), 7.0, dtype=torch.bfloat16, device="cuda")
    mx.mxfp8_gemm_bias(None, None, None, None, to_dev_bf16(bias), c, N, 40, N, 0, BIAS_EPI[epi])
    torch.cuda.synchronize()
    bv = bf16_to_f64(bias)[None, :]
    want = {"plain": bv, "gelu": oracle.gelu_epilogue(bv), "swiglu": oracle.swiglu_epilogue(bv)}[epi]
    got = bf16_to_f64(to_host(c))
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-30)


def test_grouped_uniform_counts():
    grouped_case(1024, 256, 512, [128] * 8, 3)


def test_grouped_ragged_and_empty():
    grouped_case(2048, 320, 384, [0, 320, 0, 0, 736, 32, 960, 0], 5)


def test_grouped_unaligned_counts_and_uncovered_tail():
    grouped_case(1200, 96, 256, [5, 0, 131, 257, 600], 6)   # rows 993.. belong to no group


def test_grouped_accumulate():
    grouped_case(1200, 96, 256, [5, 0, 131, 257, 600], 8, accumulate=True)


def test_grouped_decreasing_offsets_never_overlap():
    """Offsets that decrease or leave [0, M]: each bound is clamped into
    [0, M] and raised to the largest bound before it, so groups never
    overlap (a decreasing group is empty).  The result equals the oracle's
    grouped GEMM on those effective bounds, and rows outside them are not
    written."""
    torch = need_gpu()
    M, N, K = 256, 96, 256
    raw = np.array([-5, 100, 50, 200, 170, 300, 260], dtype=np.int32)
    G = len(raw) - 1
    eff = np.maximum.accumulate(np.clip(raw.astype(np.int64), 0, M))
    assert eff.tolist() == [0, 100, 100, 200, 200, 256, 256]
    x = workloads.normal_bf16((M, K), 71)
    w = workloads.normal_bf16((G, N, K), 72, std=0.02)
    qx, sx, px = quantize_on_gpu(x)
    wq = quantize_on_gpu(w.reshape(G * N, K))
    out = torch.full((M, N), -7.0, dtype=torch.bfloat16, device="cuda")
    log("grouped decreasing offsets %s" % raw.tolist())
    mx.grouped_gemm(qx, px, wq[0].view(G, N, K), wq[2], to_dev(raw), out=out)
    torch.cuda.synchronize()
    c = to_host(out)
    oqx, osx = oracle.quantize_rowwise(x)
    oq = [oracle.quantize_rowwise(w[g]) for g in range(G)]
    ref = oracle.grouped_gemm_tn(oqx, osx, np.stack([q for q, _ in oq]), np.stack([s for _, s in oq]), eff)
    gemm_tolerance_check(c, ref, K, label="grouped decreasing offsets")


def test_grouped_many_experts():
    """More experts than a wave's 64 lanes (the device-side group search walks
    the offsets 64 groups at a time): 200 ragged groups, empty ones among them
    (around the 64-group chunk boundaries too), unaligned counts, and rows
    past the last group left untouched."""
    rng = np.random.default_rng(17)
    counts = rng.integers(0, 90, size=200)
    counts[[0, 63, 64, 65, 127, 128, 199]] = 0
    counts[rng.choice(200, size=30, replace=False)] = 0
    counts[10] = 300                                   # a group spanning two row tiles
    M = int(counts.sum()) + 40
    grouped_case(M, 96, 256, list(counts), 19)


def test_grouped_single_group_matches_dense():
    grouped_case(512, 128, 256, [512], 7)


def test_grouped_empty_total():
    torch = need_gpu()
    off = to_dev(np.zeros(5, dtype=np.int32))
    c = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    mx.mxfp8_grouped_gemm(None, None, None, None, off, 4, c, 64, 0, 64, 128)


# ------------------------------------------------------ full workload sizes
#
# Every entry of every full-size output is compared with the oracle (fp64 in
# row panels), with rms over the whole output: a misplaced or skipped tile of
# the XCD / L2-group tile remap cannot hide between samples.

PANEL = 2048


def full_dense(qa, pa, qb, pb, oq_a, oq_b, K, label, excl=None):
    """GPU GEMM of device operands against the oracle's GEMM of its own
    quantizations (oq_a, oq_b = (codes, scales)) on every entry."""
    log("%s M=%d N=%d K=%d (every entry)" % (label, qa.shape[0], qb.shape[0], K))
    c = gemm_gpu(qa, pa, qb, pb)
    ref = oracle.gemm_tn(*oq_a, *oq_b, panel=PANEL)
    return gemm_full_check(c, ref, K, excl=excl, label=label, panel=PANEL)


@pytest.mark.slow
def test_full_dense_linear():
    d = workloads.dense_linear()
    qa, _, pa = quantize_on_gpu(d["X"])
    qb, _, pb = quantize_on_gpu(d["W"])
    full_dense(qa, pa, qb, pb, oracle.quantize_rowwise(d["X"]), oracle.quantize_rowwise(d["W"]), 4096,
               "dense 8192x14336x4096")


@pytest.mark.slow
def test_full_dense_linear_gelu_epilogue():
    """The dense linear GEMM 8192x14336x4096 with the GELU epilogue (an MLP's
    first projection written as GELU(X W^T)) on every entry, rms over the
    whole output."""
    d = workloads.dense_linear()
    qa, _, pa = quantize_on_gpu(d["X"])
    qb, _, pb = quantize_on_gpu(d["W"])
    log("gelu epilogue 8192x14336x4096 (every entry)")
    c = gemm_gpu(qa, pa, qb, pb, flags=mx.MXFP8_GEMM_GELU)
    ref = oracle.gemm_tn(*oracle.quantize_rowwise(d["X"]), *oracle.quantize_rowwise(d["W"]), panel=PANEL)
    rms = whole_output_rms(ref, panel=PANEL)
    for r0 in range(0, ref.shape[0], PANEL):
        gelu_tolerance_check(c[r0:r0 + PANEL], ref[r0:r0 + PANEL], 4096, label="gelu epilogue", rms=rms)


@pytest.mark.slow
def test_full_dense_square():
    d = workloads.dense_square()
    qa, _, pa = quantize_on_gpu(d["A"])
    qb, _, pb = quantize_on_gpu(d["B"])
    full_dense(qa, pa, qb, pb, oracle.quantize_rowwise(d["A"]), oracle.quantize_rowwise(d["B"]), 8192,
               "dense 8192^3")


@pytest.mark.slow
def test_full_backward_wgrad():
    d = workloads.backward()
    qa, _, pa = quantize_on_gpu(d["dY"], colwise=True)    # [4096][16384]
    qb, _, pb = quantize_on_gpu(d["X"], colwise=True)     # [4096][16384]
    full_dense(qa, pa, qb, pb, oracle.quantize_colwise(d["dY"]), oracle.quantize_colwise(d["X"]), 16384,
               "wgrad 4096x4096x16384")


@pytest.mark.slow
def test_full_stress():
    """Stress GEMM 32768x8192x8192 on every entry.  Entries whose term
    magnitudes reach 2^127 are excluded from the tolerance and from rms; the
    rows that can hold them are found from the scale bytes (a rigorous bound)
    and their magnitudes come from the oracle.  The excluded count is checked
    against a count made from the input alone: a row's max-BF16 inputs
    quantize to 448 * 2^119 = 1.75 * 2^127 (the rest of their block flushes to
    zero), so an entry is excluded when 1.75 * 2^127 * sum |dq(b)| over those
    positions, plus at most the row's other terms, reaches 2^127."""
    d = workloads.stress()
    a, b = d["A"], d["B"]
    K = a.shape[1]
    oqa, osa = oracle.quantize_rowwise(a)
    oqb, osb = oracle.quantize_rowwise(b)
    hot = overflow_candidate_rows(osa, osb, K)
    max_rows = np.unique(np.nonzero((a & 0x7FFF) == workloads.BF16_MAX_BITS)[0])
    assert set(max_rows.tolist()) <= set(hot.tolist()) and len(max_rows) > 0
    excl = np.zeros((a.shape[0], b.shape[0]), dtype=bool)
    mag = oracle.gemm_tn_abs(oqa, osa, oqb, osb, rows=hot)
    excl[hot] = mag >= 2.0 ** 127
    qa, _, pa = quantize_on_gpu(a)
    qb, _, pb = quantize_on_gpu(b)
    n_ex = full_dense(qa, pa, qb, pb, (oqa, osa), (oqb, osb), K, "stress 32768x8192x8192", excl=excl)
    # independent count from the max-BF16 positions of the input
    db_abs = np.abs(oracle.dequantize(oqb, osb))
    other = (osa.astype(np.float64), osb.astype(np.float64))
    lo = hi = 0
    for m in max_rows:
        pos = np.nonzero((a[m] & 0x7FFF) == workloads.BF16_MAX_BITS)[0]
        big = 1.75 * 2.0 ** 127 * db_abs[:, pos].sum(axis=1)
        blocks_with_max = set((pos // 32).tolist())
        rest_bytes = [other[0][m, j] for j in range(K // 32) if j not in blocks_with_max]
        rest = K * 448.0 * 448.0 * 2.0 ** ((max(rest_bytes) if rest_bytes else 0) + other[1].max() - 254.0)
        lo += int(np.sum(big >= 2.0 ** 127))
        hi += int(np.sum(big + rest >= 2.0 ** 127))
    log("stress: %d entries excluded for overflow (independent count %d..%d)" % (n_ex, lo, hi))
    assert lo <= n_ex <= hi and n_ex > 0


def _moe_refs(x, w, off):
    G = w.shape[0]
    oqx, osx = oracle.quantize_rowwise(x)
    ws = [oracle.quantize_rowwise(w[g]) for g in range(G)]
    return oracle.grouped_gemm_tn(oqx, osx, np.stack([q for q, _ in ws]), np.stack([s for _, s in ws]), off,
                                  panel=PANEL)


@pytest.mark.slow
def test_full_moe():
    torch = need_gpu()
    d = workloads.moe()
    x, w, off = d["X"], d["W"], d["offsets"]
    G, N, K = w.shape
    qx, sx, px = quantize_on_gpu(x)
    wq = quantize_on_gpu(w.reshape(G * N, K))
    log("moe grouped 16384x14336x4096 counts=%s (every entry)" % np.diff(off).tolist())
    c = to_host(mx.grouped_gemm(qx, px, wq[0].view(G, N, K), wq[2], to_dev(off)))
    torch.cuda.synchronize()
    ref = _moe_refs(x, w, off)
    assert off[0] == 0 and off[-1] == x.shape[0] and not np.isnan(ref).any()
    gemm_full_check(c, ref, K, label="moe", panel=PANEL)


@pytest.mark.slow
def test_full_moe_sqrelu():
    """The MoE first projection with the relu^2 epilogue as the benchmark runs
    it (operands quantized into packed scales), every entry."""
    torch = need_gpu()
    d = workloads.moe()
    x, w, off = d["X"], d["W"], d["offsets"]
    G, N, K = w.shape
    px_ = mx.quantize(to_dev_bf16(x), packed=True)
    pw_ = mx.quantize(to_dev_bf16(w.reshape(G * N, K)), packed=True)
    log("moe relu^2 grouped 16384x14336x4096 (every entry)")
    c = to_host(mx.grouped_gemm(px_["q_row"], px_["p_row"], pw_["q_row"].view(G, N, K), pw_["p_row"],
                                to_dev(off), sqrelu=True))
    torch.cuda.synchronize()
    ref = _moe_refs(x, w, off)
    rms = whole_output_rms(ref, panel=PANEL)
    for r0 in range(0, ref.shape[0], PANEL):
        sqrelu_tolerance_check(c[r0:r0 + PANEL], ref[r0:r0 + PANEL], K, label="moe relu^2", rms=rms)


@pytest.mark.slow
def test_full_moe_swiglu():
    """The MoE first projection with the SwiGLU epilogue at full size: X
    [16384 x 4096], each expert's 14336 rows as 7168 gate rows then 7168 up
    rows, C [16384 x 7168] = SiLU(X W_gate^T) * (X W_up^T) per expert; every
    entry, rms over the whole 14336-wide product."""
    data = workloads.moe()
    G, NB, K = data["W"].shape
    N = NB // 2
    x, w, off = data["X"], data["W"], data["offsets"]
    qx, _, px = quantize_on_gpu(x)
    wq = quantize_on_gpu(w.reshape(G * NB, K))
    log("full moe swiglu %dx%dx%d G=%d (every entry)" % (x.shape[0], N, K, G))
    c = to_host(mx.grouped_gemm(qx, px, wq[0].view(G, NB, K), wq[2], to_dev(off), swiglu=True))
    ref = _moe_refs(x, w, off)
    rms = whole_output_rms(ref, panel=PANEL)
    for r0 in range(0, ref.shape[0], PANEL):
        swiglu_tolerance_check(c[r0:r0 + PANEL], ref[r0:r0 + PANEL], K, label="moe swiglu", rms=rms)


@pytest.mark.slow
def test_full_linear_wgrad_accumulate():
    """The linear step's wgrad with accumulation at its full size
    (14336 x 4096, K = 8192 tokens) on the transposed copies, every entry."""
    torch = need_gpu()
    lin = workloads.dense_linear()
    x = lin["X"]                                        # [8192][4096]
    dy = workloads.normal_bf16((8192, 14336), 4)        # [8192][14336]
    qa, sa, pa = quantize_on_gpu(dy, colwise=True)      # [14336][8192]
    qb, sb, pb = quantize_on_gpu(x, colwise=True)       # [4096][8192]
    c_old = workloads.normal_bf16((14336, 4096), 13, std=8.0)
    cd = to_dev_bf16(c_old)
    log("wgrad accumulate 14336x4096x8192 (every entry)")
    mx.gemm(qa, pa, qb, pb, out=cd, accumulate=True)
    torch.cuda.synchronize()
    ref = oracle.gemm_tn(*oracle.quantize_colwise(dy), *oracle.quantize_colwise(x), panel=PANEL)
    ref += bf16_to_f64(c_old)
    gemm_full_check(to_host(cd), ref, 8192, label="wgrad accumulate", panel=PANEL)


@pytest.mark.slow
def test_full_linear_dgrad():
    """The linear step's dgrad at its full size (8192 x 4096, K = 14336, the
    reduction of the MLP's second projection too): dY rowwise times W's
    transposed copy, every entry."""
    need_gpu()
    w = workloads.dense_linear()["W"]                   # [14336][4096]
    dy = workloads.normal_bf16((8192, 14336), 4)        # [8192][14336]
    qa, _, pa = quantize_on_gpu(dy)                     # [8192][14336]
    qb, _, pb = quantize_on_gpu(w, colwise=True)        # [4096][14336]
    full_dense(qa, pa, qb, pb, oracle.quantize_rowwise(dy), oracle.quantize_colwise(w), 14336,
               "dgrad 8192x4096x14336")


def test_side_stream_pipeline_matches_default_stream():
    """The whole path (quantize into packed scales, GEMM) enqueued on a
    non-default stream, ordered after the input upload by an event, gives the
    same bytes as on the default stream: every launch goes to the stream it is
    given."""
    torch = need_gpu()
    a = workloads.normal_bf16((512, 640), 41)
    b = workloads.normal_bf16((384, 640), 42, std=0.05)
    xa, xb = to_dev_bf16(a), to_dev_bf16(b)
    ref_qa = mx.quantize(xa, packed=True)
    ref_qb = mx.quantize(xb, packed=True)
    ref = mx.gemm(ref_qa["q_row"], ref_qa["p_row"], ref_qb["q_row"], ref_qb["p_row"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    ready = torch.cuda.Event()
    ready.record(torch.cuda.current_stream())
    side.wait_event(ready)
    with torch.cuda.stream(side):
        qa = mx.quantize(xa, packed=True, stream=side)
        qb = mx.quantize(xb, packed=True, stream=side)
        c = mx.gemm(qa["q_row"], qa["p_row"], qb["q_row"], qb["p_row"], stream=side)
    side.synchronize()
    assert torch.equal(qa["q_row"], ref_qa["q_row"]) and torch.equal(qa["p_row"], ref_qa["p_row"])
    assert torch.equal(c.view(torch.int16), ref.view(torch.int16))
