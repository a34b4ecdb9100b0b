"""GPU tests of the GEMMs with an MXFP8 output (mxfp8_gemm_mxfp8_out,
mxfp8_grouped_gemm_mxfp8_out): the codes and packed scale words must be the
rowwise MXFP8 copy of the BF16 output the same GEMM writes otherwise.

Three kinds of check:
* against the oracle, exactly, where the BF16 output is exact (small-integer
  operands and biases: every product, sum and bias add is exact in fp32 and
  BF16), so the expected codes are the oracle's quantization of the exact
  product;
* against the oracle within the GEMM bound (any operands): each scale byte
  and code lies between those of the exact value -+ the bound of the BF16
  output (the bounded check of the activation tests);
* between the two GPU entry points, bit for bit: the fused output equals
  mxfp8_quantize_ex (ROWWISE | PACKED_SCALES) of the BF16 output of the same
  GEMM (its contract; the BF16 GEMM itself is checked against the oracle in
  test_gpu_gemm.py)."""

import numpy as np
import pytest

import mxfp8_block_scaled_quantize_amd as mx
import oracle
import workloads
from gpu_util import log, need_gpu, to_dev, to_dev_bf16, to_host
from test_gpu_gemm import product_bound, quantize_on_gpu
from test_gpu_quantize_ex import check_bounded_copy, unpack_words

pytestmark = pytest.mark.gpu

EPI = {"plain": 0, "sqrelu": mx.MXFP8_GEMM_SQRELU, "gelu": mx.MXFP8_GEMM_GELU, "swiglu": mx.MXFP8_GEMM_SWIGLU}


def words(t):
    return np.ascontiguousarray(to_host(t)).view(np.uint32)


def fused_and_unfused(qa, pa, qb, pb, M, N, K, epi, bias=None, ldq=None, offsets=None, G=0):
    """Run the MXFP8-output GEMM (with canaries around the codes and a
    padded row stride) and the BF16 GEMM + rowwise packed quantize on the same
    operands; returns (codes, words) of both and the BF16 output."""
    torch = need_gpu()
    flags = EPI[epi]
    ldq = N if ldq is None else ldq
    GD = 4096
    qbuf = torch.full((M * ldq + 2 * GD,), 0x5A, dtype=torch.uint8, device="cuda")
    q = qbuf[GD:GD + M * ldq]
    p = torch.full((N // 128, M), 0x3C3C3C3C, dtype=torch.int32, device="cuda")
    c = torch.full((M, N), 0.0, dtype=torch.bfloat16, device="cuda")
    if offsets is None:
        mx.mxfp8_gemm_mxfp8_out(qa, pa, qb, pb, bias, q, ldq, p, M, N, K, flags)
        if bias is None:
            mx.mxfp8_gemm_ex(qa, pa, qb, pb, c, N, M, N, K, flags)
        else:
            mx.mxfp8_gemm_bias(qa, pa, qb, pb, bias, c, N, M, N, K, flags)
    else:
        mx.mxfp8_grouped_gemm_mxfp8_out(qa, pa, qb, pb, offsets, G, bias, q, ldq, p, M, N, K, flags)
        if bias is None:
            mx.mxfp8_grouped_gemm_ex(qa, pa, qb, pb, offsets, G, c, N, M, N, K, flags)
        else:
            mx.mxfp8_grouped_gemm_bias(qa, pa, qb, pb, offsets, G, bias, c, N, M, N, K, flags)
    torch.cuda.synchronize()
    hq = to_host(qbuf)
    assert np.all(hq[:GD] == 0x5A) and np.all(hq[-GD:] == 0x5A), "codes written outside their rows"
    codes = hq[GD:GD + M * ldq].reshape(M, ldq)
    assert np.all(codes[:, N:] == 0x5A), "codes written beyond N"
    ref = mx.quantize(c, rowwise=True, packed=True)
    return (codes[:, :N], words(p)), (to_host(ref["q_row"]), words(ref["p_row"])), to_host(c)


@pytest.mark.parametrize("epi", ["plain", "sqrelu", "gelu", "swiglu"])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("M,N,K", [(300, 256, 512), (64, 128, 128), (513, 384, 256)])
def test_fused_equals_quantized_bf16_output(M, N, K, epi, with_bias):
    torch = need_gpu()
    NB = 2 * N if epi == "swiglu" else N
    seed = 7 * M + 11 * N + K + (1 if with_bias else 0)
    a = workloads.normal_bf16((M, K), seed)
    b = workloads.normal_bf16((NB, K), seed + 1, std=0.25)
    qa, _, pa = quantize_on_gpu(a)
    qb, _, pb = quantize_on_gpu(b)
    bias = to_dev_bf16(workloads.normal_bf16((NB,), seed + 2, std=2.0)) if with_bias else None
    log("mxfp8 out %s bias=%d M=%d N=%d K=%d" % (epi, with_bias, M, N, K))
    (q, p), (rq, rp), _ = fused_and_unfused(qa, pa, qb, pb, M, N, K, epi, bias, ldq=N + 32)
    assert np.array_equal(q, rq), "codes differ from the quantized BF16 output"
    assert np.array_equal(p, rp), "scale words differ from the quantized BF16 output"


def test_fused_within_the_gemm_bound_of_the_oracle():
    """Any operands: every scale byte and code lies between those of the
    exact product -+ the bound of the BF16 output (the GEMM bound t plus the
    BF16 rounding)."""
    M, N, K = 320, 384, 1024
    a = workloads.normal_bf16((M, K), 41)
    b = workloads.normal_bf16((N, K), 42, std=0.25)
    qa, _, pa = quantize_on_gpu(a)
    qb, _, pb = quantize_on_gpu(b)
    log("mxfp8 out vs oracle bound M=%d N=%d K=%d" % (M, N, K))
    (q, p), _, _ = fused_and_unfused(qa, pa, qb, pb, M, N, K, "plain")
    oqa, osa = oracle.quantize_rowwise(a)
    oqb, osb = oracle.quantize_rowwise(b)
    r = oracle.gemm_tn(oqa, osa, oqb, osb)
    t = product_bound(r, K)
    e = t + 2.0 ** -8 * (np.abs(r) + t)
    s = unpack_words(p, M)
    check_bounded_copy(q, s, r, e, "mxfp8 out")


@pytest.mark.parametrize("epi", ["plain", "sqrelu"])
def test_fused_exact_on_integers(epi):
    """Integer operands in {-1, 0, 1} and integer biases: R + b is an exact
    small integer, and so is relu(R + b)^2 (sparser operands keep it below
    256, where every integer is a BF16 value; checked), so the codes and words
    equal the oracle's rowwise quantization of the exact result, packed."""
    rng = np.random.default_rng(17 if epi == "plain" else 18)
    M, N, K = 200, 256, 128
    keep = 1.0 if epi == "plain" else 0.2
    A = rng.integers(-1, 2, size=(M, K)) * (rng.random((M, K)) < keep)
    B = rng.integers(-1, 2, size=(N, K)) * (rng.random((N, K)) < keep)
    bias = rng.integers(-4, 5, size=N)
    to_bits = lambda v: (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    qa, _, pa = quantize_on_gpu(to_bits(A))
    qb, _, pb = quantize_on_gpu(to_bits(B))
    log("mxfp8 out integers %s" % epi)
    (q, p), _, _ = fused_and_unfused(qa, pa, qb, pb, M, N, K, epi, to_dev_bf16(to_bits(bias)))
    exact = A @ B.T + bias[None, :]
    if epi == "sqrelu":
        exact = np.maximum(exact, 0) ** 2
    assert np.abs(exact).max() < 256                   # every value exact in BF16
    oq, os_ = oracle.quantize_rowwise(to_bits(exact))
    assert np.array_equal(q, oq)
    assert np.array_equal(p, np.ascontiguousarray(oracle.pack_scales(os_)).view(np.uint32))


def test_fused_k_zero_quantizes_the_epilogue_of_the_bias():
    """K = 0 with a bias: every row is epi(bias); plain: the oracle's rowwise
    quantization of the bias on every row."""
    torch = need_gpu()
    M, N = 96, 256
    bias = workloads.normal_bf16((N,), 44, std=3.0)
    q = torch.zeros((M, N), dtype=torch.uint8, device="cuda")
    p = torch.zeros((N // 128, M), dtype=torch.int32, device="cuda")
    mx.mxfp8_gemm_mxfp8_out(None, None, None, None, to_dev_bf16(bias), q, N, p, M, N, 0, 0)
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_rowwise(np.tile(bias, (M, 1)))
    assert np.array_equal(to_host(q), oq)
    assert np.array_equal(words(p), np.ascontiguousarray(oracle.pack_scales(os_)).view(np.uint32))


@pytest.mark.parametrize("epi", ["plain", "gelu", "swiglu"])
def test_grouped_fused_equals_quantized_bf16_output(epi):
    """Ragged experts (an empty one, group sizes not multiples of 32) and
    rows after the last group: covered rows equal the quantized BF16 output,
    uncovered rows keep their canaries (codes and scale words)."""
    torch = need_gpu()
    counts = [130, 0, 257, 64, 301]
    tail = 45
    G, N, K = len(counts), 256, 384
    M = sum(counts) + tail
    NB = 2 * N if epi == "swiglu" else N
    x = workloads.normal_bf16((M, K), 51)
    w = workloads.normal_bf16((G, NB, K), 52, std=0.05)
    qx, _, px = quantize_on_gpu(x)
    wq = quantize_on_gpu(w.reshape(G * NB, K))
    off = workloads.offsets_from_counts(counts)
    bias = to_dev_bf16(workloads.normal_bf16((G, NB), 53, std=1.0))
    log("grouped mxfp8 out %s counts=%s tail=%d" % (epi, counts, tail))
    (q, p), (rq, rp), _ = fused_and_unfused(qx, px, wq[0].view(G, NB, K), wq[2], M, N, K, epi, bias,
                                            ldq=N + 16, offsets=to_dev(off), G=G)
    rows = np.arange(off[0], off[-1])
    assert np.array_equal(q[rows], rq[rows]) and np.array_equal(p[:, rows], rp[:, rows])
    assert np.all(q[off[-1]:] == 0x5A) and np.all(p[:, off[-1]:] == 0x3C3C3C3C), "uncovered rows written"


def test_helper_returns_codes_and_words():
    """mx.gemm(..., mxfp8_out=True) returns the same arrays as the entry point."""
    need_gpu()
    M, N, K = 128, 256, 256
    a = workloads.normal_bf16((M, K), 61)
    b = workloads.normal_bf16((N, K), 62, std=0.25)
    qa, _, pa = quantize_on_gpu(a)
    qb, _, pb = quantize_on_gpu(b)
    q, p = mx.gemm(qa, pa, qb, pb, gelu=True, mxfp8_out=True)
    (fq, fp), _, _ = fused_and_unfused(qa, pa, qb, pb, M, N, K, "gelu")
    assert np.array_equal(to_host(q), fq) and np.array_equal(words(p), fp)


def test_full_size_mlp_fc1_gelu():
    """The GELU MLP's first projection at full size (8192 x 14336 x 4096, the
    inference-forward workload of bench.py): fused output equals the quantized
    BF16 output on every entry (the BF16 GELU output itself is checked
    against the oracle in test_gpu_gemm.py)."""
    need_gpu()
    lin = workloads.mlp()
    T, D = lin["X"].shape
    F = lin["W1"].shape[0]
    qx, _, px = quantize_on_gpu(lin["X"])
    qw, _, pw = quantize_on_gpu(lin["W1"])
    log("mxfp8 out full size fc1 gelu %dx%dx%d" % (T, F, D))
    (q, p), (rq, rp), _ = fused_and_unfused(qx, px, qw, pw, T, F, D, "gelu")
    assert np.array_equal(q, rq) and np.array_equal(p, rp)


def test_full_size_moe_fc1_swiglu():
    """The MoE block's first projection at full size (16384 routed rows, 8
    experts of 7168 gate + 7168 up rows, K = 4096, the moe_fwd workload of
    bench.py): the grouped fused output equals the quantized BF16 output on
    every entry (the BF16 SwiGLU output is checked against the oracle in
    test_gpu_gemm.py)."""
    need_gpu()
    d = workloads.moe()
    G, NB, K = d["W"].shape
    M = d["X"].shape[0]
    qx, _, px = quantize_on_gpu(d["X"])
    wq = quantize_on_gpu(d["W"].reshape(G * NB, K))
    log("mxfp8 out full size moe fc1 swiglu %dx%dx%d G=%d" % (M, NB, K, G))
    (q, p), (rq, rp), _ = fused_and_unfused(qx, px, wq[0].view(G, NB, K), wq[2], M, NB // 2, K, "swiglu",
                                            offsets=to_dev(d["offsets"]), G=G)
    assert np.array_equal(q, rq) and np.array_equal(p, rp)
