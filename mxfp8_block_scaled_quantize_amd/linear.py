"""MXFP8 linear layer wired through the block-scaled GEMM.

    fprop   y  = x W^T + b  TN GEMM: A = x rowwise [M][K],   B = W rowwise [N][K],
                            the optional BF16 bias b [N] added by the GEMM's bias epilogue
    dgrad   dx = dy W       TN GEMM: A = dy rowwise [M][N],  B = W columnwise copy [K][N]
    wgrad   dW = dy^T x     TN GEMM: A = dy columnwise copy [N][M], B = x columnwise copy [K][M]
    bgrad   db = sum_m dy   the dbias fused into the quantization of dy (no extra pass)

The columnwise copies are stored transposed, so every GEMM reduces over the
contiguous dimension of both operands and runs on the same TN kernel; each
quantization writes the rowwise and the transposed copy in one pass (the
MXFP8 linear flow the FlyDSL backend page validates through te.Linear: forward,
dgrad from W's columnwise copy, wgrad from the columnwise copies of dy and x).
With fuse_wgrad_accumulation the weight gradient is added to ``weight.main_grad``
(a BF16 buffer the caller owns) by the GEMM's accumulate epilogue instead of
being returned.

Shapes: x [M, K], W [N, K] BF16 with M, N and K multiples of 128 (each of the
three GEMMs reduces over one of them).

``MXFP8Linear`` keeps the weight's quantization (both copies) between calls
and quantizes the weight again only when the parameter changes: its storage,
shape or version counter (every in-place update, an optimizer step included,
bumps the counter).  Micro-batches between two weight updates reuse one
quantization.  Only the copies a GEMM will read are made: without any
gradient (grad mode off, or no input that requires one) the module's forward
quantizes the input rowwise only; x's columnwise copy is made only when the
weight needs a gradient, dy's rowwise copy only for dgrad and its columnwise
copy only for wgrad.
"""

import torch

from . import gemm, quantize


def _quantize_both(t, dbias=False):
    # one pass writes both copies with their scales already in the GEMM's
    # packed word layout (rows and columns are multiples of 128 here), and
    # with dbias=True the fp32 column sums as well
    out = quantize(t, rowwise=True, colwise=True, packed=True, dbias=dbias)
    q = (out["q_row"], out["p_row"], out["q_colT"], out["p_colT"])
    return q + (out["dbias"],) if dbias else q


def _quantize_copies(t, row, col, dbias=False):
    """Only the copies a later GEMM reads (at least one of them; dbias needs a
    copy too): (q_row, p_row, q_colT, p_colT, dbias), None where not made."""
    row = row or not col
    out = quantize(t, rowwise=row, colwise=col, packed=True, dbias=dbias)
    return out.get("q_row"), out.get("p_row"), out.get("q_colT"), out.get("p_colT"), out.get("dbias")


def _check_linear(x, weight, bias):
    """dtype and shape rules of the MXFP8 linear layer; returns the leading
    shape, the input as a contiguous [M, K] matrix, M, K and N."""
    if x.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("MXFP8 linear takes BF16 input and weight")
    if bias is not None and (bias.dtype != torch.bfloat16 or tuple(bias.shape) != (weight.shape[0],)):
        raise ValueError("bias must be a BF16 tensor with one value per output feature")
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1]).contiguous()
    M, K = x2.shape
    N = weight.shape[0]
    if weight.shape[1] != K:
        raise ValueError("weight is [%d, %d], input has %d features" % (weight.shape[0], weight.shape[1], K))
    if M % 128 or N % 128 or K % 128:
        raise ValueError("MXFP8 linear needs tokens, in- and out-features to be multiples of 128 "
                         "(got M=%d, K=%d, N=%d)" % (M, K, N))
    return lead, x2, M, K, N


def mxfp8_linear_inference(x, weight, weight_q=None, bias=None):
    """y = x W^T (+ b) without autograd: the input is quantized rowwise only
    (into packed scales) and the fprop GEMM reads the weight's rowwise copy
    (weight_q as for MXFP8LinearFunction, else the rowwise copy is made
    here)."""
    lead, x2, M, K, N = _check_linear(x, weight, bias)
    xq = quantize(x2, rowwise=True, packed=True)
    if weight_q is None:   # only the rowwise copy is read here
        wq = quantize(weight.contiguous(), rowwise=True, packed=True)
        weight_q = (wq["q_row"], wq["p_row"])
    y = gemm(xq["q_row"], xq["p_row"], weight_q[0], weight_q[1], bias=None if bias is None else bias.contiguous())
    return y.view(*lead, N)


class MXFP8LinearFunction(torch.autograd.Function):
    """apply(x, weight, fuse_wgrad_accumulation=False, weight_q=None, bias=None):
    weight_q, when given, is the weight's quantization (q_row, p_row, q_colT,
    p_colT) as ``quantize(weight, rowwise=True, colwise=True, packed=True)``
    returns it, made from the current value of ``weight``; bias, when given,
    is a BF16 [N] tensor added by the GEMM (its gradient is the fp32 dbias of
    dy's quantization, returned in the bias's dtype)."""

    @staticmethod
    def forward(ctx, x, weight, fuse_wgrad_accumulation=False, weight_q=None, bias=None):
        lead, x2, M, K, N = _check_linear(x, weight, bias)
        # x's columnwise copy only feeds wgrad
        qx, px, qxT, pxT, _ = _quantize_copies(x2, True, ctx.needs_input_grad[1])
        if weight_q is None:
            weight_q = _quantize_both(weight.contiguous())
        qw, pw, qwT, pwT = weight_q
        y = gemm(qx, px, qw, pw, bias=None if bias is None else bias.contiguous())
        ctx.save_for_backward(qxT, pxT, qwT, pwT)
        ctx.bias_dtype = None if bias is None else bias.dtype
        ctx.weight = weight
        ctx.fuse = fuse_wgrad_accumulation
        ctx.shape = (lead, M, K, N)
        return y.view(*lead, N)

    @staticmethod
    def backward(ctx, dy):
        qxT, pxT, qwT, pwT = ctx.saved_tensors
        lead, M, K, N = ctx.shape
        dy2 = dy.reshape(M, N).to(torch.bfloat16).contiguous()
        want_db = ctx.bias_dtype is not None and ctx.needs_input_grad[4]
        if not (ctx.needs_input_grad[0] or ctx.needs_input_grad[1] or want_db):
            return None, None, None, None, None
        # dy's rowwise copy feeds dgrad, its columnwise copy wgrad
        qd, pd, qdT, pdT, db = _quantize_copies(dy2, ctx.needs_input_grad[0], ctx.needs_input_grad[1], want_db)
        dx = None
        if ctx.needs_input_grad[0]:
            dx = gemm(qd, pd, qwT, pwT).view(*lead, K)
        dw = None
        if ctx.needs_input_grad[1]:
            if ctx.fuse:
                main = getattr(ctx.weight, "main_grad", None)
                if main is None or main.dtype != torch.bfloat16 or tuple(main.shape) != (N, K):
                    raise ValueError("fuse_wgrad_accumulation needs weight.main_grad, a BF16 [N, K] tensor")
                gemm(qdT, pdT, qxT, pxT, out=main, accumulate=True)
            else:
                dw = gemm(qdT, pdT, qxT, pxT)
        dbias = db.to(ctx.bias_dtype) if want_db else None
        return dx, dw, None, None, dbias


class MXFP8Linear(torch.nn.Module):
    """y = x W^T (+ b) with MXFP8 block-scaled fprop, dgrad and wgrad; the
    optional BF16 bias is added by the fprop GEMM and its gradient comes from
    the dbias fused into dy's quantization."""

    def __init__(self, in_features, out_features, fuse_wgrad_accumulation=False, device=None, bias=False):
        super().__init__()
        self.in_features, self.out_features = in_features, out_features
        self.fuse_wgrad_accumulation = fuse_wgrad_accumulation
        w = torch.empty((out_features, in_features), dtype=torch.bfloat16, device=device)
        torch.nn.init.normal_(w, std=in_features ** -0.5)
        self.weight = torch.nn.Parameter(w)
        self.bias = (torch.nn.Parameter(torch.zeros(out_features, dtype=torch.bfloat16, device=device))
                     if bias else None)
        if fuse_wgrad_accumulation:
            self.weight.main_grad = torch.zeros_like(w)
        self._wq_key = None
        self._wq = None

    def quantized_weight(self):
        """Both MXFP8 copies of the weight, quantized again only when the
        parameter's storage, shape or version counter has changed."""
        w = self.weight
        key = (w.data_ptr(), w.device, tuple(w.shape), w._version)
        if self._wq is None or self._wq_key != key:
            with torch.no_grad():
                self._wq = _quantize_both(w.detach().contiguous())
            self._wq_key = key
        return self._wq

    def forward(self, x):
        params = [self.weight] + ([self.bias] if self.bias is not None else [])
        if not (torch.is_grad_enabled() and (x.requires_grad or any(p.requires_grad for p in params))):
            return mxfp8_linear_inference(x, self.weight, self.quantized_weight(), self.bias)
        return MXFP8LinearFunction.apply(x, self.weight, self.fuse_wgrad_accumulation, self.quantized_weight(),
                                         self.bias)
