"""Python binding of libmxfp8 (MXFP8 quantize + block-scaled GEMM on gfx950).

The ``mxfp8_*`` functions mirror the C ABI of ``include/mxfp8.h`` one to one:
they only marshal arguments (torch tensors -> device pointers, torch streams
-> hipStream_t) and raise :class:`MXFP8Error` on a non-OK status.  Every step
of the computation runs in the HIP kernels of ``libmxfp8.so``; there is no
CPU fallback, and importing functions that need the library raises when it
has not been built.  PyTorch is used for device memory and streams only.

The small helpers below them (``quantize``, ``pack_scales``, ``gemm``,
``grouped_gemm``) allocate outputs with torch and call the same entry points.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxfp8.so")

MXFP8_ROWWISE = 1
MXFP8_COLWISE = 2
MXFP8_DBIAS = 4
MXFP8_AMAX = 8
MXFP8_PACKED_SCALES = 16
MXFP8_ACT_SQRELU = 32
MXFP8_DACT_SQRELU = 64
MXFP8_ACT_GELU = 128
MXFP8_DACT_GELU = 256
MXFP8_GEMM_ACCUMULATE = 1
MXFP8_GEMM_SQRELU = 2
MXFP8_GEMM_GELU = 4
MXFP8_GEMM_SWIGLU = 8
MXFP8_NOALLOC_SCRATCH_BYTES = 8 << 20

STATUS_NAMES = {0: "MXFP8_OK", 1: "MXFP8_ERR_NULL", 2: "MXFP8_ERR_SHAPE", 3: "MXFP8_ERR_MISALIGNED",
                4: "MXFP8_ERR_FLAGS", 5: "MXFP8_ERR_WORKSPACE", 6: "MXFP8_ERR_HIP", 7: "MXFP8_ERR_LIMIT"}

EXPORTED = ("mxfp8_status_string", "mxfp8_last_hip_error", "mxfp8_quantize_workspace_bytes",
            "mxfp8_quantize", "mxfp8_packed_scale_bytes", "mxfp8_pack_scales", "mxfp8_gemm",
            "mxfp8_grouped_gemm", "mxfp8_gemm_ex", "mxfp8_grouped_gemm_ex", "mxfp8_gemm_bias",
            "mxfp8_grouped_gemm_bias", "mxfp8_gemm_mxfp8_out", "mxfp8_grouped_gemm_mxfp8_out", "mxfp8_quantize_ex",
            "mxfp8_quantize_ex_noalloc")


class MXFP8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().mxfp8_status_string(status).decode()
        if status == 6:
            msg += " (hipError %d)" % lib().mxfp8_last_hip_error()
        super().__init__("%s: %s" % (where, msg))


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmxfp8.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmxfp8.so is not built (run mxfp8_block_scaled_quantize_amd.build.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, U32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    L.mxfp8_status_string.restype = ctypes.c_char_p
    L.mxfp8_status_string.argtypes = [ctypes.c_int]
    L.mxfp8_last_hip_error.restype = ctypes.c_int
    L.mxfp8_last_hip_error.argtypes = []
    L.mxfp8_quantize_workspace_bytes.restype = SZ
    L.mxfp8_quantize_workspace_bytes.argtypes = [I64, I64, U32]
    L.mxfp8_quantize.restype = ctypes.c_int
    L.mxfp8_quantize.argtypes = [P, I64, I64, I64, U32, P, P, P, P, P, P, SZ, P]
    L.mxfp8_packed_scale_bytes.restype = SZ
    L.mxfp8_packed_scale_bytes.argtypes = [I64, I64]
    L.mxfp8_pack_scales.restype = ctypes.c_int
    L.mxfp8_pack_scales.argtypes = [P, I64, I64, I64, P, P]
    L.mxfp8_gemm.restype = ctypes.c_int
    L.mxfp8_gemm.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P]
    L.mxfp8_grouped_gemm.restype = ctypes.c_int
    L.mxfp8_grouped_gemm.argtypes = [P, P, P, P, P, I32, P, I64, I64, I64, I64, P]
    L.mxfp8_quantize_ex.restype = ctypes.c_int
    L.mxfp8_quantize_ex.argtypes = [P, I64, I64, I64, U32, P, P, P, P, P, P, P, P, P, SZ, P]
    L.mxfp8_quantize_ex_noalloc.restype = ctypes.c_int
    L.mxfp8_quantize_ex_noalloc.argtypes = [P, I64, I64, I64, U32, P, P, P, P, P, P, P, P, P]
    L.mxfp8_gemm_ex.restype = ctypes.c_int
    L.mxfp8_gemm_ex.argtypes = [P, P, P, P, P, I64, I64, I64, I64, U32, P]
    L.mxfp8_grouped_gemm_ex.restype = ctypes.c_int
    L.mxfp8_grouped_gemm_ex.argtypes = [P, P, P, P, P, I32, P, I64, I64, I64, I64, U32, P]
    L.mxfp8_gemm_bias.restype = ctypes.c_int
    L.mxfp8_gemm_bias.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, U32, P]
    L.mxfp8_grouped_gemm_bias.restype = ctypes.c_int
    L.mxfp8_grouped_gemm_bias.argtypes = [P, P, P, P, P, I32, P, P, I64, I64, I64, I64, U32, P]
    L.mxfp8_gemm_mxfp8_out.restype = ctypes.c_int
    L.mxfp8_gemm_mxfp8_out.argtypes = [P, P, P, P, P, P, I64, P, I64, I64, I64, U32, P]
    L.mxfp8_grouped_gemm_mxfp8_out.restype = ctypes.c_int
    L.mxfp8_grouped_gemm_mxfp8_out.argtypes = [P, P, P, P, P, I32, P, P, I64, P, I64, I64, I64, U32, P]
    _lib = L
    return L


def _p(t):
    """Device pointer of a tensor (or an int address, or None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream):
    """hipStream_t of a torch stream (None -> torch's current stream)."""
    if isinstance(stream, int):
        return stream
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise MXFP8Error(status, where)


# ------------------------------------------------------------ C ABI mirror

def mxfp8_status_string(status: int) -> str:
    return lib().mxfp8_status_string(status).decode()


def mxfp8_last_hip_error() -> int:
    return lib().mxfp8_last_hip_error()


def mxfp8_quantize_workspace_bytes(rows: int, cols: int, flags: int) -> int:
    return lib().mxfp8_quantize_workspace_bytes(rows, cols, flags)


def mxfp8_quantize(x, rows, cols, ld_x, flags, q_row=None, s_row=None, q_colT=None, s_colT=None,
                   dbias=None, workspace=None, workspace_bytes=0, stream=None):
    _check(lib().mxfp8_quantize(_p(x), rows, cols, ld_x, flags, _p(q_row), _p(s_row), _p(q_colT),
                                _p(s_colT), _p(dbias), _p(workspace), workspace_bytes, _s(stream)),
           "mxfp8_quantize")


def mxfp8_quantize_ex(x, rows, cols, ld_x, flags, q_row=None, s_row=None, q_colT=None, s_colT=None,
                      dbias=None, amax=None, noop=None, act_in=None, workspace=None, workspace_bytes=0,
                      stream=None):
    _check(lib().mxfp8_quantize_ex(_p(x), rows, cols, ld_x, flags, _p(q_row), _p(s_row), _p(q_colT),
                                   _p(s_colT), _p(dbias), _p(amax), _p(noop), _p(act_in), _p(workspace),
                                   workspace_bytes, _s(stream)), "mxfp8_quantize_ex")


def mxfp8_quantize_ex_noalloc(x, rows, cols, ld_x, flags, q_row=None, s_row=None, q_colT=None, s_colT=None,
                              dbias=None, amax=None, noop=None, act_in=None, stream=None):
    _check(lib().mxfp8_quantize_ex_noalloc(_p(x), rows, cols, ld_x, flags, _p(q_row), _p(s_row), _p(q_colT),
                                           _p(s_colT), _p(dbias), _p(amax), _p(noop), _p(act_in), _s(stream)),
           "mxfp8_quantize_ex_noalloc")


def mxfp8_packed_scale_bytes(dim: int, k: int) -> int:
    return lib().mxfp8_packed_scale_bytes(dim, k)


def mxfp8_pack_scales(s, dim, k, ld_s, packed, stream=None):
    _check(lib().mxfp8_pack_scales(_p(s), dim, k, ld_s, _p(packed), _s(stream)), "mxfp8_pack_scales")


def mxfp8_gemm(a, a_packed, b, b_packed, c, ldc, M, N, K, stream=None):
    _check(lib().mxfp8_gemm(_p(a), _p(a_packed), _p(b), _p(b_packed), _p(c), ldc, M, N, K, _s(stream)),
           "mxfp8_gemm")


def mxfp8_grouped_gemm(a, a_packed, b, b_packed, offsets, G, c, ldc, M_total, N, K, stream=None):
    _check(lib().mxfp8_grouped_gemm(_p(a), _p(a_packed), _p(b), _p(b_packed), _p(offsets), G, _p(c), ldc,
                                    M_total, N, K, _s(stream)), "mxfp8_grouped_gemm")


def mxfp8_gemm_ex(a, a_packed, b, b_packed, c, ldc, M, N, K, flags, stream=None):
    _check(lib().mxfp8_gemm_ex(_p(a), _p(a_packed), _p(b), _p(b_packed), _p(c), ldc, M, N, K, flags, _s(stream)),
           "mxfp8_gemm_ex")


def mxfp8_gemm_bias(a, a_packed, b, b_packed, bias, c, ldc, M, N, K, flags, stream=None):
    _check(lib().mxfp8_gemm_bias(_p(a), _p(a_packed), _p(b), _p(b_packed), _p(bias), _p(c), ldc, M, N, K, flags,
                                 _s(stream)), "mxfp8_gemm_bias")


def mxfp8_grouped_gemm_bias(a, a_packed, b, b_packed, offsets, G, bias, c, ldc, M_total, N, K, flags, stream=None):
    _check(lib().mxfp8_grouped_gemm_bias(_p(a), _p(a_packed), _p(b), _p(b_packed), _p(offsets), G, _p(bias), _p(c),
                                         ldc, M_total, N, K, flags, _s(stream)), "mxfp8_grouped_gemm_bias")


def mxfp8_gemm_mxfp8_out(a, a_packed, b, b_packed, bias, q_out, ldq, q_out_packed, M, N, K, flags, stream=None):
    _check(lib().mxfp8_gemm_mxfp8_out(_p(a), _p(a_packed), _p(b), _p(b_packed), _p(bias), _p(q_out), ldq,
                                      _p(q_out_packed), M, N, K, flags, _s(stream)), "mxfp8_gemm_mxfp8_out")


def mxfp8_grouped_gemm_mxfp8_out(a, a_packed, b, b_packed, offsets, G, bias, q_out, ldq, q_out_packed, M_total, N,
                                 K, flags, stream=None):
    _check(lib().mxfp8_grouped_gemm_mxfp8_out(_p(a), _p(a_packed), _p(b), _p(b_packed), _p(offsets), G, _p(bias),
                                              _p(q_out), ldq, _p(q_out_packed), M_total, N, K, flags, _s(stream)),
           "mxfp8_grouped_gemm_mxfp8_out")


def mxfp8_grouped_gemm_ex(a, a_packed, b, b_packed, offsets, G, c, ldc, M_total, N, K, flags, stream=None):
    _check(lib().mxfp8_grouped_gemm_ex(_p(a), _p(a_packed), _p(b), _p(b_packed), _p(offsets), G, _p(c), ldc,
                                       M_total, N, K, flags, _s(stream)), "mxfp8_grouped_gemm_ex")


# ------------------------------------------------------ allocating helpers

def quantize(x, rowwise=True, colwise=False, dbias=False, amax=False, packed=False, noop=None, act=None,
             act_in=None, stream=None):
    """Quantize a BF16 [rows, cols] CUDA tensor; returns a dict of outputs.

    packed=True returns the scales in the packed word layout ("p_row" int32
    [cols/128, rows], "p_colT" int32 [rows/128, cols]) instead of bytes;
    amax=True adds "amax" (fp32 [1]); noop is an optional int32 tensor on x's
    device whose first element is the flag (nonzero: nothing is written).
    act="sqrelu" quantizes relu(x)^2; act="dsqrelu" quantizes
    x * 2 relu(act_in) (x is the gradient, act_in the activation's input, a
    BF16 tensor of x's shape and strides); act="gelu" quantizes GELU(x) and
    act="dgelu" x * GELU'(act_in) (GELU(x) = x Phi(x), not the tanh approximation; fp32)."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a BF16 [rows, cols] tensor with unit column stride")
    if x.device.type != "cuda":
        raise ValueError("x must be a CUDA (HIP) tensor, got %s" % x.device)
    R, C = x.shape
    dev = x.device
    if noop is not None and (not isinstance(noop, torch.Tensor) or noop.dtype != torch.int32
                             or noop.device != dev or noop.numel() < 1):
        raise ValueError("noop must be an int32 tensor with at least one element on x's device (%s)" % dev)
    flags = (MXFP8_ROWWISE if rowwise else 0) | (MXFP8_COLWISE if colwise else 0) | (MXFP8_DBIAS if dbias else 0)
    flags |= (MXFP8_AMAX if amax else 0) | (MXFP8_PACKED_SCALES if packed else 0)
    acts = {"sqrelu": MXFP8_ACT_SQRELU, "dsqrelu": MXFP8_DACT_SQRELU, "gelu": MXFP8_ACT_GELU,
            "dgelu": MXFP8_DACT_GELU}
    if act is not None and act not in acts:
        raise ValueError("act must be None or one of %s" % ", ".join(repr(k) for k in acts))
    if act in ("dsqrelu", "dgelu"):
        if (act_in is None or act_in.dtype != torch.bfloat16 or act_in.shape != x.shape
                or act_in.stride() != x.stride() or act_in.device != x.device):
            raise ValueError("act=%r needs act_in: a BF16 tensor with x's shape, strides and device" % act)
    if act is not None:
        flags |= acts[act]
    out = {}
    if rowwise:
        out["q_row"] = torch.empty((R, C), dtype=torch.uint8, device=dev)
        if packed:
            out["p_row"] = torch.empty((C // 128, R), dtype=torch.int32, device=dev)
        else:
            out["s_row"] = torch.empty((R, C // 32), dtype=torch.uint8, device=dev)
    if colwise:
        out["q_colT"] = torch.empty((C, R), dtype=torch.uint8, device=dev)
        if packed:
            out["p_colT"] = torch.empty((R // 128, C), dtype=torch.int32, device=dev)
        else:
            out["s_colT"] = torch.empty((C, R // 32), dtype=torch.uint8, device=dev)
    ws = None
    nws = mxfp8_quantize_workspace_bytes(R, C, flags)
    if dbias:
        out["dbias"] = torch.empty((C,), dtype=torch.float32, device=dev)
    if amax:
        out["amax"] = torch.empty((1,), dtype=torch.float32, device=dev)
    if nws:
        ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
    s_row = out.get("p_row") if packed else out.get("s_row")
    s_col = out.get("p_colT") if packed else out.get("s_colT")
    with torch.cuda.device(dev):
        if amax or packed or noop is not None or act is not None:
            mxfp8_quantize_ex(x, R, C, x.stride(0), flags, out.get("q_row"), s_row, out.get("q_colT"), s_col,
                              out.get("dbias"), out.get("amax"), noop, act_in, ws, nws, stream)
        else:
            mxfp8_quantize(x, R, C, x.stride(0), flags, out.get("q_row"), s_row, out.get("q_colT"), s_col,
                           out.get("dbias"), ws, nws, stream)
    return out


def _require(t, name, dtype, shape=None, device=None):
    """Host-side checks of a tensor handed to the C ABI as a dense array."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a CUDA (HIP) tensor, got %s" % (name, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def pack_scales(s, stream=None):
    """E8M0 scales uint8 [dim, K/32] -> packed int32 words [K/128, dim]."""
    import torch
    if not isinstance(s, torch.Tensor) or s.dtype != torch.uint8 or s.dim() != 2 or s.stride(1) != 1:
        raise ValueError("s must be a uint8 [dim, K/32] tensor with unit column stride")
    if s.device.type != "cuda":
        raise ValueError("s must be a CUDA (HIP) tensor, got %s" % s.device)
    dim, kb = s.shape
    out = torch.empty((kb // 4, dim), dtype=torch.int32, device=s.device)
    with torch.cuda.device(s.device):
        mxfp8_pack_scales(s, dim, kb * 32, s.stride(0), out, stream)
    return out


def _gemm_flags(accumulate, sqrelu, gelu, swiglu=False):
    if accumulate + sqrelu + gelu + swiglu > 1:
        raise ValueError("accumulate, sqrelu, gelu and swiglu exclude each other")
    return ((MXFP8_GEMM_ACCUMULATE if accumulate else 0) | (MXFP8_GEMM_SQRELU if sqrelu else 0)
            | (MXFP8_GEMM_GELU if gelu else 0) | (MXFP8_GEMM_SWIGLU if swiglu else 0))


def gemm(a, a_packed, b, b_packed, out=None, accumulate=False, sqrelu=False, gelu=False, swiglu=False,
         bias=None, mxfp8_out=False, stream=None):
    """C = dq(A) dq(B)^T in BF16 for E4M3 codes a [M, K], b [N, K]; with
    accumulate=True the product is added to `out` (beta = 1); with
    sqrelu=True C = relu(product)^2, with gelu=True C = GELU(product)
    (formed in fp32, rounded once).  swiglu=True: b is [2N, K] (gate rows,
    then up rows) and C [M, N] = SiLU(gate product) * up product.  bias (a
    BF16 tensor with one value per row of b) is added to the fp32 product
    before the activation (not with accumulate).  mxfp8_out=True returns C's
    rowwise MXFP8 copy instead, as (codes uint8 [M, N], packed scale words
    int32 [N / 128, M]) (N % 128 == 0; not with accumulate or out)."""
    import torch
    if not isinstance(a, torch.Tensor) or a.dim() != 2 or not isinstance(b, torch.Tensor) or b.dim() != 2:
        raise ValueError("a and b must be 2-D tensors of E4M3 codes")
    M, K = a.shape
    NB = b.shape[0]
    if swiglu and NB % 2:
        raise ValueError("swiglu=True needs b with an even number of rows (gate rows, then up rows)")
    N = NB // 2 if swiglu else NB
    dev = a.device
    _require(a, "a", torch.uint8)
    _require(b, "b", torch.uint8, (NB, K), dev)
    _require(a_packed, "a_packed", torch.int32, (K // 128, M), dev)
    _require(b_packed, "b_packed", torch.int32, (K // 128, NB), dev)
    if accumulate and out is None:
        raise ValueError("accumulate=True needs out")
    c = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if c.dtype != torch.bfloat16 or tuple(c.shape) != (M, N) or c.stride(1) != 1 or c.device != dev:
        raise ValueError("out must be a BF16 [M, N] tensor with unit column stride on the operands' device")
    flags = _gemm_flags(accumulate, sqrelu, gelu, swiglu)
    if bias is not None:
        if accumulate:
            raise ValueError("bias and accumulate exclude each other")
        _require(bias, "bias", torch.bfloat16, (NB,), dev)
    if mxfp8_out:
        return _mx_out(M, N, dev, accumulate, out, lambda q, p: mxfp8_gemm_mxfp8_out(
            a, a_packed, b, b_packed, bias, q, N, p, M, N, K, flags, stream))
    with torch.cuda.device(dev):
        if bias is not None:
            mxfp8_gemm_bias(a, a_packed, b, b_packed, bias, c, c.stride(0), M, N, K, flags, stream)
        else:
            mxfp8_gemm_ex(a, a_packed, b, b_packed, c, c.stride(0), M, N, K, flags, stream)
    return c


def _mx_out(M, N, dev, accumulate, out, call):
    """Allocate the MXFP8 output of a GEMM and run `call(codes, packed)`."""
    import torch
    if accumulate or out is not None:
        raise ValueError("mxfp8_out=True writes fresh outputs: no accumulate, no out")
    if N % 128:
        raise ValueError("mxfp8_out=True needs N % 128 == 0 (whole packed scale words)")
    q = torch.zeros((M, N), dtype=torch.uint8, device=dev)
    p = torch.zeros((N // 128, M), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        call(q, p)
    return q, p


def grouped_gemm(a, a_packed, b, b_packed, offsets, out=None, accumulate=False, sqrelu=False, gelu=False,
                 swiglu=False, bias=None, mxfp8_out=False, stream=None):
    """Ragged grouped GEMM; b is [G, N, K]; rows outside every group keep `out`'s values;
    sqrelu=True writes relu(product)^2 (an MoE block's first projection), gelu=True GELU(product);
    swiglu=True: b is [G, 2N, K] (per expert gate rows, then up rows), C [M, N] = SiLU(gate) * up;
    bias: BF16 [G, rows of an expert], added per expert before the activation; mxfp8_out=True:
    (codes [M, N], packed scale words [N / 128, M]) as for gemm, rows outside every group left
    unwritten (zero in freshly allocated outputs)."""
    import torch
    if not isinstance(a, torch.Tensor) or a.dim() != 2 or not isinstance(b, torch.Tensor) or b.dim() != 3:
        raise ValueError("a must be 2-D [M, K] and b 3-D [G, N, K] tensors of E4M3 codes")
    M, K = a.shape
    G, NB, _ = b.shape
    if swiglu and NB % 2:
        raise ValueError("swiglu=True needs experts with an even number of rows (gate rows, then up rows)")
    N = NB // 2 if swiglu else NB
    dev = a.device
    _require(a, "a", torch.uint8)
    _require(b, "b", torch.uint8, (G, NB, K), dev)
    _require(a_packed, "a_packed", torch.int32, (K // 128, M), dev)
    _require(b_packed, "b_packed", torch.int32, (K // 128, G * NB), dev)
    _require(offsets, "offsets", torch.int32, (G + 1,), dev)
    if accumulate and out is None:
        raise ValueError("accumulate=True needs out")
    flags = _gemm_flags(accumulate, sqrelu, gelu, swiglu)
    if bias is not None:
        if accumulate:
            raise ValueError("bias and accumulate exclude each other")
        _require(bias, "bias", torch.bfloat16, (G, NB), dev)
    if mxfp8_out:
        return _mx_out(M, N, dev, accumulate, out, lambda q, p: mxfp8_grouped_gemm_mxfp8_out(
            a, a_packed, b, b_packed, offsets, G, bias, q, N, p, M, N, K, flags, stream))
    c = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if c.dtype != torch.bfloat16 or tuple(c.shape) != (M, N) or c.stride(1) != 1 or c.device != dev:
        raise ValueError("out must be a BF16 [M, N] tensor with unit column stride on the operands' device")
    with torch.cuda.device(dev):
        if bias is not None:
            mxfp8_grouped_gemm_bias(a, a_packed, b, b_packed, offsets, G, bias, c, c.stride(0), M, N, K, flags,
                                    stream)
        else:
            mxfp8_grouped_gemm_ex(a, a_packed, b, b_packed, offsets, G, c, c.stride(0), M, N, K, flags, stream)
    return c
