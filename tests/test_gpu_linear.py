"""MXFP8 linear layer (fprop, dgrad, wgrad and fused wgrad accumulation) on
the GPU path, against the oracle's GEMMs of its own quantizations of the same
BF16 tensors (rowwise copies for fprop, the transposed columnwise copies for
dgrad and wgrad), and loosely against plain fp32 PyTorch."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import bf16_to_f64, gemm_tolerance_check, log, need_gpu, to_dev_bf16, to_host

pytestmark = pytest.mark.gpu

M, K, N = 256, 384, 512


def _inputs(seed):
    x = workloads.normal_bf16((M, K), seed)
    w = workloads.normal_bf16((N, K), seed + 1, std=0.05)
    dy = workloads.normal_bf16((M, N), seed + 2)
    return x, w, dy


def _refs(x, w, dy):
    qx, sx = oracle.quantize_rowwise(x)
    qw, sw = oracle.quantize_rowwise(w)
    y = oracle.gemm_tn(qx, sx, qw, sw)
    qd, sd = oracle.quantize_rowwise(dy)
    qwT, swT = oracle.quantize_colwise(w)
    dx = oracle.gemm_tn(qd, sd, qwT, swT)
    qdT, sdT = oracle.quantize_colwise(dy)
    qxT, sxT = oracle.quantize_colwise(x)
    dw = oracle.gemm_tn(qdT, sdT, qxT, sxT)
    return y, dx, dw


def _run(x, w, dy, fuse=False, main_grad=None):
    torch = need_gpu()
    from mxfp8_block_scaled_quantize_amd.linear import MXFP8LinearFunction
    xt = to_dev_bf16(x).requires_grad_(True)
    wt = to_dev_bf16(w).requires_grad_(True)
    if fuse:
        wt.main_grad = main_grad
    y = MXFP8LinearFunction.apply(xt, wt, fuse)
    y.backward(to_dev_bf16(dy))
    torch.cuda.synchronize()
    return y.detach(), xt.grad, wt.grad


def test_linear_fprop_dgrad_wgrad_match_oracle():
    x, w, dy = _inputs(30)
    log("linear M=%d K=%d N=%d" % (M, K, N))
    y, dx, dw = _run(x, w, dy)
    y_ref, dx_ref, dw_ref = _refs(x, w, dy)
    gemm_tolerance_check(to_host(y), y_ref, K, label="fprop")
    gemm_tolerance_check(to_host(dx), dx_ref, N, label="dgrad")
    gemm_tolerance_check(to_host(dw), dw_ref, M, label="wgrad")


def test_linear_close_to_fp32_pytorch():
    torch = need_gpu()
    x, w, dy = _inputs(31)
    y, dx, dw = _run(x, w, dy)
    xf = torch.from_numpy(bf16_to_f64(x))
    wf = torch.from_numpy(bf16_to_f64(w))
    dyf = torch.from_numpy(bf16_to_f64(dy))
    for got, want, name in ((y, xf @ wf.T, "y"), (dx, dyf @ wf, "dx"), (dw, dyf.T @ xf, "dw")):
        g = torch.from_numpy(bf16_to_f64(to_host(got)))
        rel = (torch.linalg.norm(g - want) / torch.linalg.norm(want)).item()
        log("%s relative error vs fp32: %.4f" % (name, rel))
        assert rel < 0.08, (name, rel)   # MXFP8 (3 mantissa bits) on both operands


def test_linear_fused_wgrad_accumulation():
    torch = need_gpu()
    x, w, dy = _inputs(32)
    g0 = workloads.normal_bf16((N, K), 99, std=3.0)
    main = to_dev_bf16(g0)
    _, _, dw = _run(x, w, dy, fuse=True, main_grad=main)
    assert dw is None
    _, _, dw_ref = _refs(x, w, dy)
    got1 = to_host(main).copy()
    gemm_tolerance_check(got1, dw_ref + bf16_to_f64(g0), M, label="accumulate 1")
    dy2 = workloads.normal_bf16((M, N), 77)
    _run(x, w, dy2, fuse=True, main_grad=main)
    _, _, dw2_ref = _refs(x, w, dy2)
    # The second step adds to the BF16 result of the first.  Against the host
    # values only: |final - (dW1 + dW2 + g0)| <= t1 + t2 (the GEMM bound of
    # each product) plus the two BF16 roundings, 2^-9 of the first sum and of
    # the final value (doubled for margin).
    def bound(ref):
        return 8e-3 * np.abs(ref) + 1e-3 * np.sqrt(M) * np.sqrt(np.mean(ref ** 2))
    t1, t2 = bound(dw_ref), bound(dw2_ref)
    want = dw_ref + dw2_ref + bf16_to_f64(g0)
    first = np.abs(dw_ref + bf16_to_f64(g0)) + t1
    tol = t1 + t2 + 2.0 ** -8 * first + 2.0 ** -8 * (np.abs(want) + t1 + t2 + 2.0 ** -8 * first)
    err = np.abs(bf16_to_f64(to_host(main)) - want)
    assert np.all(err <= tol), "accumulate 2: %d entries out of tolerance" % np.sum(err > tol)


def test_linear_module_reuses_weight_quantization_until_the_weight_changes(monkeypatch):
    """MXFP8Linear quantizes W once per weight value: a second forward with an
    unchanged weight launches only the input's quantize; an in-place update
    (as an optimizer step does) makes the next forward quantize W again.
    Outputs match the oracle on the current weight each time."""
    torch = need_gpu()
    import mxfp8_block_scaled_quantize_amd.linear as lin
    calls = []
    real = lin.quantize

    def counting(t, **kw):
        calls.append(tuple(t.shape))
        return real(t, **kw)

    monkeypatch.setattr(lin, "quantize", counting)
    x1, w, _ = _inputs(33)
    x2 = workloads.normal_bf16((M, K), 34)
    layer = lin.MXFP8Linear(K, N, device="cuda")
    with torch.no_grad():
        layer.weight.copy_(to_dev_bf16(w))
    log("linear module weight cache")
    for i, x in enumerate((x1, x2)):
        y = layer(to_dev_bf16(x))
        torch.cuda.synchronize()
        qx, sx = oracle.quantize_rowwise(x)
        qw, sw = oracle.quantize_rowwise(w)
        gemm_tolerance_check(to_host(y), oracle.gemm_tn(qx, sx, qw, sw), K, label="forward %d" % i)
    assert calls == [(N, K), (M, K), (M, K)], calls      # W quantized once (first), x twice
    w2 = workloads.normal_bf16((N, K), 35, std=0.05)
    with torch.no_grad():
        layer.weight.copy_(to_dev_bf16(w2))              # in-place: bumps the version counter
    del calls[:]
    y = layer(to_dev_bf16(x1))
    torch.cuda.synchronize()
    assert calls == [(N, K), (M, K)], calls
    qx, sx = oracle.quantize_rowwise(x1)
    qw, sw = oracle.quantize_rowwise(w2)
    gemm_tolerance_check(to_host(y), oracle.gemm_tn(qx, sx, qw, sw), K, label="forward after update")


def _bias_checks(y, db, x, w, dy, bias, label):
    """y = x W^T + b against the oracle's product plus the bias (the GEMM bound
    of the unbiased product, plus the BF16 rounding of the biased value);
    the bias gradient against the oracle's column sums of dy (the fp32 dbias
    bound of the quantize tests, plus its rounding to BF16, 2^-9 doubled)."""
    from test_gpu_quantize import dbias_depth
    y_ref, _, _ = _refs(x, w, dy)
    t = 8e-3 * np.abs(y_ref) + 1e-3 * np.sqrt(K) * np.sqrt(np.mean(y_ref ** 2))
    want = oracle.bias_add(y_ref, bias)
    err = np.abs(bf16_to_f64(to_host(y)) - want)
    tol = t + 2.0 ** -8 * (np.abs(want) + t)
    assert np.all(err <= tol), "%s fprop: %d entries out of tolerance" % (label, np.sum(err > tol))
    ref = oracle.dbias(dy).astype(np.float64)
    mag = np.abs(bf16_to_f64(dy)).sum(axis=0)
    tol = 1.01 * dbias_depth(M) * 2.0 ** -24 * mag + np.abs(ref) * 2.0 ** -24 + 2.0 ** -126
    tol = tol + 2.0 ** -8 * (np.abs(ref) + tol)
    err = np.abs(bf16_to_f64(to_host(db)) - ref)
    assert np.all(err <= tol), "%s dbias off by %g" % (label, err.max())


def test_linear_with_bias():
    """The bias goes through the GEMM's bias epilogue in fprop and its gradient
    through the dbias fused into dy's quantization; dgrad and wgrad are the
    same as without a bias."""
    torch = need_gpu()
    from mxfp8_block_scaled_quantize_amd.linear import MXFP8LinearFunction
    x, w, dy = _inputs(36)
    bias = workloads.normal_bf16((N,), 37, std=1.0)
    log("linear with bias M=%d K=%d N=%d" % (M, K, N))
    xt = to_dev_bf16(x).requires_grad_(True)
    wt = to_dev_bf16(w).requires_grad_(True)
    bt = to_dev_bf16(bias).requires_grad_(True)
    y = MXFP8LinearFunction.apply(xt, wt, False, None, bt)
    y.backward(to_dev_bf16(dy))
    torch.cuda.synchronize()
    assert bt.grad.dtype == torch.bfloat16 and tuple(bt.grad.shape) == (N,)
    _bias_checks(y.detach(), bt.grad, x, w, dy, bias, "function")
    _, dx_ref, dw_ref = _refs(x, w, dy)
    gemm_tolerance_check(to_host(xt.grad), dx_ref, N, label="dgrad with bias")
    gemm_tolerance_check(to_host(wt.grad), dw_ref, M, label="wgrad with bias")


def test_linear_module_with_bias():
    torch = need_gpu()
    import mxfp8_block_scaled_quantize_amd.linear as lin
    x, w, dy = _inputs(38)
    bias = workloads.normal_bf16((N,), 39, std=1.0)
    layer = lin.MXFP8Linear(K, N, device="cuda", bias=True)
    with torch.no_grad():
        layer.weight.copy_(to_dev_bf16(w))
        layer.bias.copy_(to_dev_bf16(bias))
    log("linear module with bias")
    y = layer(to_dev_bf16(x))
    y.backward(to_dev_bf16(dy))
    torch.cuda.synchronize()
    _bias_checks(y.detach(), layer.bias.grad, x, w, dy, bias, "module")


def test_linear_module_inference_quantizes_the_input_rowwise_only(monkeypatch):
    """Without grad the module quantizes the input rowwise only (no columnwise
    copy: nothing reads it) and its output equals the autograd path's bit for
    bit (the same codes reach the same GEMM) and the oracle within the bound."""
    torch = need_gpu()
    import mxfp8_block_scaled_quantize_amd.linear as lin
    calls = []
    real = lin.quantize

    def recording(t, **kw):
        calls.append((tuple(t.shape), bool(kw.get("colwise"))))
        return real(t, **kw)

    monkeypatch.setattr(lin, "quantize", recording)
    x, w, dy = _inputs(40)
    bias = workloads.normal_bf16((N,), 41, std=1.0)
    layer = lin.MXFP8Linear(K, N, device="cuda", bias=True)
    with torch.no_grad():
        layer.weight.copy_(to_dev_bf16(w))
        layer.bias.copy_(to_dev_bf16(bias))
    log("linear module inference")
    xt = to_dev_bf16(x)
    with torch.no_grad():
        y_inf = layer(xt)
    torch.cuda.synchronize()
    assert calls == [((N, K), True), ((M, K), False)], calls     # W's two copies (cached), x rowwise only
    y_train = layer(xt)                                           # grad mode: the weight requires grad
    torch.cuda.synchronize()
    assert calls[2:] == [((M, K), True)], calls
    assert torch.equal(y_inf.view(torch.int16), y_train.detach().view(torch.int16))
    y_ref, _, _ = _refs(x, w, dy)
    t = 8e-3 * np.abs(y_ref) + 1e-3 * np.sqrt(K) * np.sqrt(np.mean(y_ref ** 2))
    want = oracle.bias_add(y_ref, bias)
    err = np.abs(bf16_to_f64(to_host(y_inf)) - want)
    assert np.all(err <= t + 2.0 ** -8 * (np.abs(want) + t))


@pytest.mark.parametrize("frozen", ["weight", "input"])
def test_linear_makes_only_the_copies_its_gradients_read(monkeypatch, frozen):
    """A frozen weight: x is quantized rowwise only and dy rowwise only (dgrad);
    an input that needs no gradient: dy is quantized columnwise only (wgrad).
    The gradients that are computed match the oracle."""
    torch = need_gpu()
    import mxfp8_block_scaled_quantize_amd.linear as lin
    calls = []
    real = lin.quantize

    def recording(t, **kw):
        calls.append((tuple(t.shape), bool(kw.get("rowwise", True)), bool(kw.get("colwise"))))
        return real(t, **kw)

    monkeypatch.setattr(lin, "quantize", recording)
    x, w, dy = _inputs(42)
    xt = to_dev_bf16(x).requires_grad_(frozen == "weight")
    wt = to_dev_bf16(w).requires_grad_(frozen == "input")
    log("linear frozen %s" % frozen)
    wq = lin._quantize_both(wt.detach())
    del calls[:]
    y = lin.MXFP8LinearFunction.apply(xt, wt, False, wq)
    y.backward(to_dev_bf16(dy))
    torch.cuda.synchronize()
    y_ref, dx_ref, dw_ref = _refs(x, w, dy)
    gemm_tolerance_check(to_host(y.detach()), y_ref, K, label="fprop")
    if frozen == "weight":
        assert calls == [((M, K), True, False), ((M, N), True, False)], calls
        assert wt.grad is None
        gemm_tolerance_check(to_host(xt.grad), dx_ref, N, label="dgrad")
    else:
        assert calls == [((M, K), True, True), ((M, N), False, True)], calls
        assert xt.grad is None
        gemm_tolerance_check(to_host(wt.grad), dw_ref, M, label="wgrad")
