"""A squared-ReLU MLP training step run through the library with the calls
and layouts of the MLP benchmark step: row+col quantize of X, W1, W2, dY;
FC1 GEMM; relu^2 fused into the quantize of a BF16 hidden tensor H; FC2 GEMM;
FC2 dgrad and wgrad; the activation's backward fused into the
row+col+dbias quantize of a BF16 gradient dA, which also reads H; FC1 dgrad
and wgrad.

The oracle runs the same step from the host tensors alone: its H and dA are
its own GEMM outputs rounded to BF16.  Those are uploaded as the GPU's inputs
to the activation launches, so every GPU stage is compared with the oracle on
identical inputs (no oracle input or expected value comes from the GPU):
quantize launches bit for bit, GEMMs within the GEMM tolerance, dbias within
the summation bound; the GPU's own FC1 and FC2-dgrad outputs are checked
against the oracle's H and dA within the GEMM tolerance."""

import numpy as np
import pytest

import mxfp8_block_scaled_quantize_amd as mx
import oracle
import workloads
from gpu_util import gemm_tolerance_check, log, need_gpu, to_dev_bf16, to_host

pytestmark = pytest.mark.gpu


def check_quantized(got, v):
    """Packed row+col outputs of the library against the oracle's quantization of fp32 values v."""
    q, s = oracle.quantize_rowwise_values(v)
    qT, sT = oracle.quantize_colwise_values(v)
    assert np.array_equal(to_host(got["q_row"]), q)
    assert np.array_equal(to_host(got["p_row"]), oracle.pack_scales(s))
    assert np.array_equal(to_host(got["q_colT"]), qT)
    assert np.array_equal(to_host(got["p_colT"]), oracle.pack_scales(sT))
    return (q, s), (qT, sT)


def bf16_of(r):
    """The oracle's BF16 copy of an fp64 GEMM result (fp32, then RNE to BF16)."""
    return workloads.f32_to_bf16_bits(np.asarray(r, dtype=np.float32))


@pytest.mark.parametrize("T,D,F", [(256, 256, 384), (384, 512, 640)])
def test_squared_relu_mlp_step(T, D, F):
    torch = need_gpu()
    log("mlp T=%d D=%d F=%d" % (T, D, F))
    x = workloads.normal_bf16((T, D), 61)
    w1 = workloads.normal_bf16((F, D), 62, std=0.05)
    w2 = workloads.normal_bf16((D, F), 63, std=0.05)
    dy = workloads.normal_bf16((T, D), 64)
    val = oracle.bf16_value
    f32 = lambda b: val(b).astype(np.float32)

    qx = mx.quantize(to_dev_bf16(x), rowwise=True, colwise=True, packed=True)
    qw1 = mx.quantize(to_dev_bf16(w1), rowwise=True, colwise=True, packed=True)
    (x_r, x_c) = check_quantized(qx, f32(x))
    (w1_r, w1_c) = check_quantized(qw1, f32(w1))

    # FC1: the GPU's output against the oracle's; the oracle's H feeds the rest
    h_ref = oracle.gemm_tn(*x_r, *w1_r)
    gemm_tolerance_check(to_host(mx.gemm(qx["q_row"], qx["p_row"], qw1["q_row"], qw1["p_row"])), h_ref, D,
                         label="fc1")
    h_bits = bf16_of(h_ref)
    h = to_dev_bf16(h_bits)

    qa = mx.quantize(h, rowwise=True, colwise=True, packed=True, act="sqrelu")
    a_r, a_c = check_quantized(qa, oracle.act_sqrelu(h_bits))

    qw2 = mx.quantize(to_dev_bf16(w2), rowwise=True, colwise=True, packed=True)
    w2_r, w2_c = check_quantized(qw2, f32(w2))
    y = mx.gemm(qa["q_row"], qa["p_row"], qw2["q_row"], qw2["p_row"])
    gemm_tolerance_check(to_host(y), oracle.gemm_tn(*a_r, *w2_r), F, label="fc2")

    qdy = mx.quantize(to_dev_bf16(dy), rowwise=True, colwise=True, packed=True)
    dy_r, dy_c = check_quantized(qdy, f32(dy))
    da_ref = oracle.gemm_tn(*dy_r, *w2_c)
    gemm_tolerance_check(to_host(mx.gemm(qdy["q_row"], qdy["p_row"], qw2["q_colT"], qw2["p_colT"])), da_ref, D,
                         label="fc2 dgrad")
    dw2 = mx.gemm(qdy["q_colT"], qdy["p_colT"], qa["q_colT"], qa["p_colT"])
    gemm_tolerance_check(to_host(dw2), oracle.gemm_tn(*dy_c, *a_c), T, label="fc2 wgrad")

    da_bits = bf16_of(da_ref)
    qdh = mx.quantize(to_dev_bf16(da_bits), rowwise=True, colwise=True, dbias=True, packed=True, act="dsqrelu",
                      act_in=h)
    dh = oracle.dact_sqrelu(da_bits, h_bits)
    dh_r, dh_c = check_quantized(qdh, dh)
    ref = oracle.dbias_values(dh).astype(np.float64)
    mag = np.abs(dh.astype(np.float64)).sum(axis=0)
    depth = 8 + 2 + 3 + ((T + 127) // 128 + 7) // 8 + 3
    tol = 1.01 * depth * 2.0 ** -24 * mag + np.abs(ref) * 2.0 ** -24 + 2.0 ** -126
    assert np.all(np.abs(to_host(qdh["dbias"]).astype(np.float64) - ref) <= tol)

    dx = mx.gemm(qdh["q_row"], qdh["p_row"], qw1["q_colT"], qw1["p_colT"])
    gemm_tolerance_check(to_host(dx), oracle.gemm_tn(*dh_r, *w1_c), F, label="fc1 dgrad")
    dw1 = mx.gemm(qdh["q_colT"], qdh["p_colT"], qx["q_colT"], qx["p_colT"])
    gemm_tolerance_check(to_host(dw1), oracle.gemm_tn(*dh_c, *x_c), T, label="fc1 wgrad")
    torch.cuda.synchronize()
