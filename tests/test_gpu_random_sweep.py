"""Seeded randomized parity sweeps against the oracle: quantize calls with
random shapes, leading dimensions, copy sets and extras (dbias, amax, packed
scales, fused activations), dense GEMMs with random M, N, K, ldc and epilogues,
and grouped GEMMs with random group sizes (empty and non-multiple-of-32 groups,
uncovered tails).  Each case is drawn from a fixed generator, so a failure
names a reproducible case; the checks are the same as in the hand-picked
tests (bit-exact codes and scales, dbias within its summation bound, GEMM
within the stated tolerance; GELU outputs within the bounded check of the
GELU tests).  MXFP8_SWEEP_SCALE=k in the environment multiplies every case
count by k."""

import os

import numpy as np
import pytest

import mxfp8_block_scaled_quantize_amd as mx
import oracle
import workloads
from gpu_util import bf16_to_f64, gemm_tolerance_check, log, need_gpu, to_dev_bf16, to_host
from test_gpu_gemm import (bias_case, gelu_tolerance_check, gemm_gpu, grouped_case, quantize_on_gpu,
                           sqrelu_tolerance_check, swiglu_tolerance_check)
from test_gpu_quantize_ex import act_inputs, check_act_result, check_gelu_result, dgelu_case, gelu_case, run_ex

pytestmark = pytest.mark.gpu

# MXFP8_SWEEP_SCALE=k runs k times as many cases of every sweep (the first
# ones are the default cases: each generator draws its cases in order).
SCALE = max(1, int(os.environ.get("MXFP8_SWEEP_SCALE", "1")))

ROW, COL, DB = mx.MXFP8_ROWWISE, mx.MXFP8_COLWISE, mx.MXFP8_DBIAS
AMAX, PACKED = mx.MXFP8_AMAX, mx.MXFP8_PACKED_SCALES
ACT, DACT = mx.MXFP8_ACT_SQRELU, mx.MXFP8_DACT_SQRELU


def quantize_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        flags = [ROW, COL, ROW | COL][rng.integers(0, 3)]
        flags |= DB if rng.random() < 0.35 else 0
        flags |= AMAX if rng.random() < 0.35 else 0
        flags |= PACKED if rng.random() < 0.4 else 0
        act = [0, 0, ACT, DACT][rng.integers(0, 4)]
        cmul = 128 if (flags & PACKED and flags & ROW) else 32
        rmul = 128 if (flags & PACKED and flags & COL) else (32 if flags & COL else 1)
        C = cmul * int(rng.integers(1, 1024 // cmul + 1))
        R = rmul * int(rng.integers(1, 640 // rmul + 1))
        ld = C + 8 * int(rng.integers(0, 5)) if rng.random() < 0.4 else C
        cases.append((R, C, ld, flags, act, int(rng.integers(0, 1 << 30))))
    return cases


@pytest.mark.parametrize("case", quantize_cases(48 * SCALE, 2024))
def test_random_quantize(case):
    R, C, ld, flags, act, seed = case
    label = "random quantize R=%d C=%d ld=%d flags=%d act=%d seed=%d" % case
    log(label)
    if act:
        g, a = act_inputs(R, C, seed)
        got = run_ex(g, flags | act, ld=ld, act_bits=a if act == DACT else None)
        v = oracle.act_sqrelu(g) if act == ACT else oracle.dact_sqrelu(g, a)
    else:
        # max-BF16 values only without dbias (their column sums would overflow fp32)
        bits = workloads.wide_range_bf16((R, C), seed, n_maxbf16=0 if flags & DB else 2, n_subnormal=16,
                                         n_subnormal_blocks=1)
        got = run_ex(bits, flags, ld=ld)
        v = workloads.bf16_bits_to_f32(bits)   # BF16 values quantize like their fp32 copies (pinned)
    check_act_result(got, v, flags, label)


def gemm_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        M = int(rng.integers(1, 700))
        N = 32 * int(rng.integers(1, 26))
        K = 128 * int(rng.integers(1, 13))
        ldc = N + 8 * int(rng.integers(0, 4)) if rng.random() < 0.4 else N
        epi = ["plain", "plain", "accumulate", "sqrelu"][rng.integers(0, 4)]
        cases.append((M, N, K, ldc, epi, int(rng.integers(0, 1 << 30))))
    return cases


@pytest.mark.parametrize("case", gemm_cases(32 * SCALE, 77))
def test_random_gemm(case):
    torch = need_gpu()
    M, N, K, ldc, epi, seed = case
    log("random gemm M=%d N=%d K=%d ldc=%d %s seed=%d" % case)
    a = workloads.normal_bf16((M, K), seed)
    b = workloads.normal_bf16((N, K), seed + 1, std=0.25)
    qa, sa, pa = quantize_on_gpu(a)
    qb, sb, pb = quantize_on_gpu(b)
    oqa, osa = oracle.quantize_rowwise(a)
    oqb, osb = oracle.quantize_rowwise(b)
    ref = oracle.gemm_tn(oqa, osa, oqb, osb)
    if epi == "accumulate":
        old = workloads.normal_bf16((M, ldc), seed + 2, std=3.0)
        cbuf = to_dev_bf16(old)
        mx.mxfp8_gemm_ex(qa, pa, qb, pb, cbuf, ldc, M, N, K, mx.MXFP8_GEMM_ACCUMULATE)
        torch.cuda.synchronize()
        got = to_host(cbuf)
        assert np.array_equal(got[:, N:], old[:, N:]), "columns beyond N written"
        gemm_tolerance_check(got[:, :N], ref + bf16_to_f64(old[:, :N]), K, label="accumulate")
    elif epi == "sqrelu":
        c = gemm_gpu(qa, pa, qb, pb, ldc=ldc, canary=True, flags=mx.MXFP8_GEMM_SQRELU)
        sqrelu_tolerance_check(c, ref, K, "sqrelu")
    else:
        c = gemm_gpu(qa, pa, qb, pb, ldc=ldc, canary=True)
        gemm_tolerance_check(c, ref, K, label="gemm")


def grouped_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        G = int(rng.integers(1, 13))
        counts = rng.integers(0, 400, size=G)
        counts[rng.random(G) < 0.2] = 0
        tail = int(rng.integers(0, 3)) * int(rng.integers(1, 100))   # rows after the last group
        N = 32 * int(rng.integers(1, 9))
        K = 128 * int(rng.integers(1, 5))
        epi = ["plain", "accumulate", "sqrelu"][rng.integers(0, 3)]
        cases.append((tuple(int(c) for c in counts), tail, N, K, epi, int(rng.integers(0, 1 << 20))))
    return cases


@pytest.mark.parametrize("case", grouped_cases(20 * SCALE, 91))
def test_random_grouped_gemm(case):
    counts, tail, N, K, epi, seed = case
    M = sum(counts) + tail
    if M == 0:
        pytest.skip("empty problem (covered by test_grouped_empty_total)")
    grouped_case(M, N, K, list(counts), seed, accumulate=epi == "accumulate", sqrelu=epi == "sqrelu")


GELU, DGELU = mx.MXFP8_ACT_GELU, mx.MXFP8_DACT_GELU


def gelu_quantize_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for (R, C, ld, flags, _, s) in quantize_cases(n, seed):
        cases.append((R, C, ld, flags, [GELU, DGELU][rng.integers(0, 2)], s))
    return cases


@pytest.mark.parametrize("case", gelu_quantize_cases(24 * SCALE, 2025))
def test_random_gelu_quantize(case):
    R, C, ld, flags, act, seed = case
    label = "random gelu quantize R=%d C=%d ld=%d flags=%d act=%d seed=%d" % case
    log(label)
    if act == GELU:
        x, v, e = gelu_case(R, C, seed)
        got = run_ex(x, flags | GELU, ld=ld)
    else:
        g, a, v, e = dgelu_case(R, C, seed)
        got = run_ex(g, flags | DGELU, ld=ld, act_bits=a)
    check_gelu_result(got, v, e, flags, label)


@pytest.mark.parametrize("case", gemm_cases(12 * SCALE, 78))
def test_random_gemm_gelu(case):
    M, N, K, ldc, _, seed = case
    log("random gemm gelu M=%d N=%d K=%d ldc=%d seed=%d" % (M, N, K, ldc, seed))
    a = workloads.normal_bf16((M, K), seed)
    b = workloads.normal_bf16((N, K), seed + 1, std=0.25)
    qa, sa, pa = quantize_on_gpu(a)
    qb, sb, pb = quantize_on_gpu(b)
    oqa, osa = oracle.quantize_rowwise(a)
    oqb, osb = oracle.quantize_rowwise(b)
    c = gemm_gpu(qa, pa, qb, pb, ldc=ldc, canary=True, flags=mx.MXFP8_GEMM_GELU)
    gelu_tolerance_check(c, oracle.gemm_tn(oqa, osa, oqb, osb), K, "gelu")


@pytest.mark.parametrize("case", grouped_cases(8 * SCALE, 92))
def test_random_grouped_gemm_gelu(case):
    counts, tail, N, K, _, seed = case
    M = sum(counts) + tail
    if M == 0:
        pytest.skip("empty problem (covered by test_grouped_empty_total)")
    grouped_case(M, N, K, list(counts), seed, gelu=True)


@pytest.mark.parametrize("case", gemm_cases(12 * SCALE, 79))
def test_random_gemm_swiglu(case):
    """B = [gate; up] with 2N rows, C [M, N]: random M, N (a multiple of 32,
    often not of 128), K and ldc."""
    M, N, K, ldc, _, seed = case
    log("random gemm swiglu M=%d N=%d K=%d ldc=%d seed=%d" % (M, N, K, ldc, seed))
    a = workloads.normal_bf16((M, K), seed)
    b = workloads.normal_bf16((2 * N, K), seed + 1, std=0.25)
    qa, sa, pa = quantize_on_gpu(a)
    qb, sb, pb = quantize_on_gpu(b)
    oqa, osa = oracle.quantize_rowwise(a)
    oqb, osb = oracle.quantize_rowwise(b)
    c = gemm_gpu(qa, pa, qb, pb, ldc=ldc, canary=True, flags=mx.MXFP8_GEMM_SWIGLU)
    swiglu_tolerance_check(c, oracle.gemm_tn(oqa, osa, oqb, osb), K, "swiglu")


@pytest.mark.parametrize("case", grouped_cases(8 * SCALE, 93))
def test_random_grouped_gemm_swiglu(case):
    counts, tail, N, K, _, seed = case
    M = sum(counts) + tail
    if M == 0:
        pytest.skip("empty problem (covered by test_grouped_empty_total)")
    grouped_case(M, N, K, list(counts), seed, swiglu=True)


EPIS = ["plain", "sqrelu", "gelu", "swiglu"]


@pytest.mark.parametrize("case", gemm_cases(12 * SCALE, 80))
def test_random_gemm_bias(case):
    """The bias epilogue under each activation, random M, N, K and ldc."""
    M, N, K, ldc, _, seed = case
    bias_case(M, N, K, EPIS[seed % 4], seed, ldc=ldc)


@pytest.mark.parametrize("case", grouped_cases(8 * SCALE, 94))
def test_random_grouped_gemm_bias(case):
    counts, tail, N, K, _, seed = case
    M = sum(counts) + tail
    if M == 0:
        pytest.skip("empty problem (covered by test_grouped_empty_total)")
    epi = EPIS[seed % 4]
    grouped_case(M, N, K, list(counts), seed, bias=True, sqrelu=epi == "sqrelu", gelu=epi == "gelu",
                 swiglu=epi == "swiglu")


def mxout_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        M = int(rng.integers(1, 700))
        N = 128 * int(rng.integers(1, 6))
        K = 128 * int(rng.integers(1, 9))
        ldq = N + 16 * int(rng.integers(0, 3))
        cases.append((M, N, K, ldq, EPIS[int(rng.integers(0, 4))], bool(rng.integers(0, 2)),
                      int(rng.integers(0, 1 << 30))))
    return cases


@pytest.mark.parametrize("case", mxout_cases(12 * SCALE, 81))
def test_random_gemm_mxfp8_out(case):
    """The MXFP8-output GEMM equals the rowwise packed quantize of the BF16
    output, random shapes, row strides, epilogues and biases."""
    from test_gpu_gemm_mxout import fused_and_unfused
    M, N, K, ldq, epi, with_bias, seed = case
    log("random mxfp8 out M=%d N=%d K=%d ldq=%d %s bias=%d seed=%d" % case)
    NB = 2 * N if epi == "swiglu" else N
    qa, _, pa = quantize_on_gpu(workloads.normal_bf16((M, K), seed))
    qb, _, pb = quantize_on_gpu(workloads.normal_bf16((NB, K), seed + 1, std=0.25))
    bias = to_dev_bf16(workloads.normal_bf16((NB,), seed + 2, std=1.0)) if with_bias else None
    (q, p), (rq, rp), _ = fused_and_unfused(qa, pa, qb, pb, M, N, K, epi, bias, ldq=ldq)
    assert np.array_equal(q, rq) and np.array_equal(p, rp)
