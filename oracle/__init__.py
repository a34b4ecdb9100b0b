"""CPU oracle for MXFP8 block-scaled quantization and the block-scaled GEMM.

TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only code allowed to import this package.
The product path (the HIP library and its Python binding) never calls it and
shares no code with it.

The quantizer lives in ``mx_oracle.c`` (plain C, double precision, one block
at a time).  The GEMMs are defined here: dequantize every code exactly
(E4M3 value times 2^(scale byte - 127), exact in double) and contract in
double with ``numpy.matmul``.  Each product of two dequantized values is exact
in double; only the fp64 summation rounds, far below the GEMM tolerance.

Passages followed (page titles; the pages print no worked example and no
formula for the scale rule, so the OCP MX rule is the reading taken):

* block of 32 elements along K, rowwise and columnwise copies, dbias:
  "[Common] Experimental CuTeDSL MXFP8 backends in C++ via TVM-FFI"
  (review thread on 32-divisible shapes; Greptile summary; config struct
  fields rowwise / colwise / with_dbias).
* E8M0 scale byte as a bare exponent: "frost(gemm): Add Rubin kernel
  pipelines" (nitpick on the ue8m0 readback).
* MXFP8 x MXFP8 -> BF16 TN GEMM with fp32 accumulation, alpha = 1, beta = 0,
  and the [K/128, dim] packed-scale word layout: "Experimental FlyDSL GEMM
  backend for TE PyTorch (BF16/FP16/FP32/FP8/MXFP8)" (Summary; commit notes on
  the fused scale-pack kernel; review of the epilogue validation).
* grouped GEMM over ragged row ranges given by int32 expert offsets, empty
  groups legal: "gemm(cutedsl): add standalone Lightning W4A16 grouped GEMM"
  (PR body) and "frost(gemm): Add Rubin kernel pipelines" (review of the MoE
  grouped template: per-group row base and row extent).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mx_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmx_oracle.so")
_lib = None

MX_BLOCK = 32


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (OpenMP over rows/columns only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fno-fast-math", "-fopenmp",
                               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_decode.restype = ctypes.c_double
    lib.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_scale_byte.restype = ctypes.c_uint8
    lib.oracle_scale_byte.argtypes = [ctypes.c_double]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    for name in ("oracle_quantize_rows", "oracle_quantize_cols", "oracle_quantize_rows_f32",
                 "oracle_quantize_cols_f32"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [P, I64, I64, I64, P, P]
    lib.oracle_dbias.restype = None
    lib.oracle_dbias.argtypes = [P, I64, I64, I64, P]
    lib.oracle_dbias_f32.restype = None
    lib.oracle_dbias_f32.argtypes = [P, I64, I64, I64, P]
    lib.oracle_dequantize.restype = None
    lib.oracle_dequantize.argtypes = [P, P, I64, I64, P]
    lib.oracle_e4m3_encode_array.restype = None
    lib.oracle_e4m3_encode_array.argtypes = [P, I64, P]
    lib.oracle_pack_scales.restype = None
    lib.oracle_pack_scales.argtypes = [P, I64, I64, I64, P]
    lib.oracle_scale_byte_array.restype = None
    lib.oracle_scale_byte_array.argtypes = [P, I64, P]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def num_threads() -> int:
    """Threads the C oracle's parallel loops use (OpenMP max threads)."""
    return int(_load().oracle_num_threads())


# ------------------------------------------------------------------ codecs

def e4m3_decode(codes) -> np.ndarray:
    """Exact value of E4M3 codes as float64 (NaN for 0x7F / 0xFF)."""
    lib = _load()
    table = np.array([lib.oracle_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e8m0_decode(b) -> np.ndarray:
    lib = _load()
    table = np.array([lib.oracle_e8m0_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(b, dtype=np.uint8)]


def e4m3_encode(values) -> np.ndarray:
    """Saturating round-to-nearest-even E4M3 codes of exact float64 values."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def scale_byte(amax: float) -> int:
    return int(_load().oracle_scale_byte(float(amax)))


def scale_bytes(amax) -> np.ndarray:
    """E8M0 scale bytes of an array of block amax values (same rule as scale_byte)."""
    a = np.ascontiguousarray(amax, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint8)
    _load().oracle_scale_byte_array(_ptr(a), a.size, _ptr(out))
    return out


def bf16_value(bits) -> np.ndarray:
    """BF16 bit patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------- quantize

def _check_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    if x.ndim != 2:
        raise ValueError("expected a 2-D BF16 bit-pattern array")
    if np.any((x & 0x7F80) == 0x7F80):
        raise ValueError("NaN/Inf inputs are outside the quantizer's contract")
    return x


def quantize_rowwise(x_bits: np.ndarray):
    """Rowwise MXFP8 copy: (codes uint8[R][C], scales uint8[R][C/32])."""
    x = _check_bf16(x_bits)
    R, C = x.shape
    if C % MX_BLOCK:
        raise ValueError("columns must be a multiple of 32")
    q = np.empty((R, C), dtype=np.uint8)
    s = np.empty((R, C // MX_BLOCK), dtype=np.uint8)
    _load().oracle_quantize_rows(_ptr(x), R, C, C, _ptr(q), _ptr(s))
    return q, s


def quantize_colwise(x_bits: np.ndarray):
    """Columnwise MXFP8 copy stored transposed: (codes uint8[C][R], scales uint8[C][R/32])."""
    x = _check_bf16(x_bits)
    R, C = x.shape
    if R % MX_BLOCK:
        raise ValueError("rows must be a multiple of 32 for the columnwise copy")
    qT = np.empty((C, R), dtype=np.uint8)
    sT = np.empty((C, R // MX_BLOCK), dtype=np.uint8)
    _load().oracle_quantize_cols(_ptr(x), R, C, C, _ptr(qT), _ptr(sT))
    return qT, sT


def dbias(x_bits: np.ndarray) -> np.ndarray:
    """Column sums of the unquantized BF16 input, float32[C]."""
    x = _check_bf16(x_bits)
    R, C = x.shape
    out = np.empty(C, dtype=np.float32)
    _load().oracle_dbias(_ptr(x), R, C, C, _ptr(out))
    return out


# ------------------------------------------------ activation-fused quantize
#
# The quantization config of "[Common] Experimental CuTeDSL MXFP8 backends in
# C++ via TVM-FFI" (review of the config key) has with_act / with_dact
# options; the activation this library implements is the squared ReLU that
# "gemm(cutedsl): add standalone Lightning W4A16 grouped GEMM" names as the
# FC1 epilogue (relu(x)^2).  Its value and its derivative 2 relu(a) are
# computed in fp32 exactly as a kernel does (numpy float32 arithmetic, round
# to nearest even: both products of two BF16 values are exact unless they
# leave the fp32 normal range), then quantized exactly.

def act_sqrelu(x_bits: np.ndarray) -> np.ndarray:
    """relu(x)^2 of BF16 x, in fp32."""
    x = bf16_value(_check_bf16(x_bits)).astype(np.float32)
    r = np.maximum(x, np.float32(0.0))
    return (r * r).astype(np.float32)


def dact_sqrelu(grad_bits: np.ndarray, act_bits: np.ndarray) -> np.ndarray:
    """grad * d/da relu(a)^2 = grad * (2 relu(a)), in fp32."""
    g = bf16_value(_check_bf16(grad_bits)).astype(np.float32)
    a = bf16_value(_check_bf16(act_bits)).astype(np.float32)
    two_r = np.float32(2.0) * np.maximum(a, np.float32(0.0))
    return (g * two_r).astype(np.float32)


def sqrelu_epilogue(r: np.ndarray) -> np.ndarray:
    """relu(r)^2 of a GEMM result, in fp64: the FC1 "squared_relu" epilogue of
    "gemm(cutedsl): add standalone Lightning W4A16 grouped GEMM - #811"
    (section "API and compatibility impact"), applied to the product before
    its output rounding."""
    r = np.asarray(r, dtype=np.float64)
    z = np.maximum(r, 0.0)
    return z * z


# GELU (the with_act / with_dact activation the quantization config of
# "[Common] Experimental CuTeDSL MXFP8 backends in C++ via TVM-FFI" names, and
# the fused GELU epilogue that "Experimental FlyDSL GEMM backend for TE PyTorch
# (BF16/FP16/FP32/FP8/MXFP8)" says its MXFP8 path drops).  The pages give no
# formula; the reading is the exact (erf) form GELU(x) = x Phi(x) with Phi the
# standard normal CDF, written as 0.5 x erfc(-x / sqrt(2)) so that the negative
# tail keeps its relative accuracy, and its derivative Phi(a) + a phi(a).
# Values are exact up to fp64 rounding (scipy's erfc and exp).

_SQRT1_2 = 0.7071067811865476
_INV_SQRT_2PI = 0.3989422804014327


def _erfc(z):
    from scipy.special import erfc
    return erfc(z)


def gelu_f64(x) -> np.ndarray:
    """GELU(x) = 0.5 x erfc(-x / sqrt(2)) in float64."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * _erfc(-x * _SQRT1_2)


def dgelu_terms(a):
    """The two terms of GELU'(a) = Phi(a) + a phi(a), in float64."""
    a = np.asarray(a, dtype=np.float64)
    return 0.5 * _erfc(-a * _SQRT1_2), a * np.exp(-0.5 * a * a) * _INV_SQRT_2PI


def act_gelu(x_bits: np.ndarray) -> np.ndarray:
    """GELU of BF16 inputs, float64."""
    return gelu_f64(bf16_value(_check_bf16(x_bits)))


def dact_gelu(grad_bits: np.ndarray, act_bits: np.ndarray) -> np.ndarray:
    """grad * GELU'(a) of BF16 inputs, float64."""
    t1, t2 = dgelu_terms(bf16_value(_check_bf16(act_bits)))
    return bf16_value(_check_bf16(grad_bits)) * (t1 + t2)


def gelu_epilogue(r: np.ndarray) -> np.ndarray:
    """GELU of a GEMM result (the epilogue applied before the output rounding)."""
    return gelu_f64(r)


# SwiGLU (the block-scale matmul and MoE grouped block-scale matmul forward
# with a SwiGLU epilogue that "frost(gemm): Add Rubin kernel pipelines" lists
# among its tests and benchmarks).  The pages give no formula or layout; the
# reading is the standard gated form SwiGLU = SiLU(gate) * up with
# SiLU(z) = z sigma(z) = z / (1 + exp(-z)), the GEMM's B holding the gate
# projection in its first N rows and the up projection in the next N
# (grouped: per expert), so C[m][n] = SiLU(R[m][n]) * R[m][N + n] for the
# fp64 product R = A B^T over the 2N rows.

def bias_add(r: np.ndarray, bias_bits: np.ndarray) -> np.ndarray:
    """The bias epilogue of the GEMM (the fused bias that "Experimental FlyDSL
    GEMM backend for TE PyTorch (BF16/FP16/FP32/FP8/MXFP8)" leaves as a TODO
    and that te.Linear(bias=True) needs, review of the fallback exceptions):
    R[m][n] + bias[n] in float64, the BF16 bias taken exactly, before any
    activation epilogue and the output rounding.  r [.., C], bias [C]."""
    b = bf16_value(np.asarray(bias_bits, dtype=np.uint16))
    r = np.asarray(r, dtype=np.float64)
    if b.shape != r.shape[-1:]:
        raise ValueError("bias must have one value per product column")
    return r + b


def silu_f64(z) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z)) in float64 (exp overflow for z < -709
    gives z / inf = -0, the correctly rounded value)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_epilogue(r: np.ndarray) -> np.ndarray:
    """SwiGLU of a GEMM result over 2N columns [gate | up] -> [.., N]."""
    r = np.asarray(r, dtype=np.float64)
    n2 = r.shape[-1]
    if n2 % 2:
        raise ValueError("SwiGLU needs an even number of product columns")
    n = n2 // 2
    return silu_f64(r[..., :n]) * r[..., n:]


def _check_f32(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    if v.ndim != 2 or v.shape[1] % MX_BLOCK:
        raise ValueError("expected [R][C] with C a multiple of 32")
    if not np.all(np.isfinite(v)):
        raise ValueError("values must be finite")
    return v


def quantize_rowwise_values(v: np.ndarray):
    """Rowwise MXFP8 copy of fp32 values: (codes uint8[R][C], scales uint8[R][C/32])."""
    v = _check_f32(v)
    R, C = v.shape
    q = np.empty((R, C), dtype=np.uint8)
    s = np.empty((R, C // MX_BLOCK), dtype=np.uint8)
    _load().oracle_quantize_rows_f32(_ptr(v), R, C, C, _ptr(q), _ptr(s))
    return q, s


def quantize_colwise_values(v: np.ndarray):
    """Columnwise MXFP8 copy of fp32 values, stored transposed."""
    v = _check_f32(v)
    R, C = v.shape
    if R % MX_BLOCK:
        raise ValueError("rows must be a multiple of 32 for the columnwise copy")
    qT = np.empty((C, R), dtype=np.uint8)
    sT = np.empty((C, R // MX_BLOCK), dtype=np.uint8)
    _load().oracle_quantize_cols_f32(_ptr(v), R, C, C, _ptr(qT), _ptr(sT))
    return qT, sT


def dbias_values(v: np.ndarray) -> np.ndarray:
    """Column sums of fp32 values (double accumulation, rounded once)."""
    v = _check_f32(v)
    R, C = v.shape
    out = np.empty(C, dtype=np.float32)
    _load().oracle_dbias_f32(_ptr(v), R, C, C, _ptr(out))
    return out


def amax(x_bits: np.ndarray) -> float:
    """Per-tensor amax: the largest |x| of the BF16 input (the with_amax output
    of the quantization config, "[Common] Experimental CuTeDSL MXFP8 backends
    in C++ via TVM-FFI", review of the config key); 0.0 for an empty tensor."""
    x = np.asarray(x_bits, dtype=np.uint16)
    if x.size == 0:
        return 0.0
    return float(np.abs(bf16_value(x)).max())


def dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """float64 values of codes q[R][C] under block scales s[R][C/32]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    R, C = q.shape
    if s.shape != (R, C // MX_BLOCK):
        raise ValueError("scale shape does not match codes")
    out = np.empty((R, C), dtype=np.float64)
    _load().oracle_dequantize(_ptr(q), _ptr(s), R, C, _ptr(out))
    return out


# ------------------------------------------------------------ scale packing

def pack_scales(s: np.ndarray) -> np.ndarray:
    """Scales s[dim][K/32] -> uint32 words packed[K/128][dim].

    Byte j (little-endian) of word (t, r) is the scale of K-block 4t + j of
    row r: one word per 128-wide K slab per row, rows contiguous within a slab.
    """
    s = np.ascontiguousarray(s, dtype=np.uint8)
    dim, kb = s.shape
    if kb % 4:
        raise ValueError("K must be a multiple of 128 (K/32 a multiple of 4)")
    out = np.empty((kb // 4, dim, 4), dtype=np.uint8)
    _load().oracle_pack_scales(_ptr(s), dim, kb, kb, _ptr(out))
    return out.view("<u4").reshape(kb // 4, dim)


# ------------------------------------------------------------------- GEMMs

def gemm_tn(qa, sa, qb, sb, rows=None, cols=None, panel=None) -> np.ndarray:
    """C[m, n] = sum_k dq(A)[m, k] * dq(B)[n, k] in float64 (TN: both K-major).

    ``rows``/``cols`` restrict the result to a sub-grid (sampled checking of
    large shapes); the entries are the same as in the full product.
    ``panel`` evaluates the product ``panel`` rows of A at a time (B is
    dequantized once), which bounds the memory of large products; each entry
    is the same sum, up to the order BLAS adds its terms in.
    """
    if rows is not None:
        qa, sa = qa[rows], sa[rows]
    if cols is not None:
        qb, sb = qb[cols], sb[cols]
    dbT = dequantize(qb, sb).T
    if panel is None or qa.shape[0] <= panel:
        return np.matmul(dequantize(qa, sa), dbT)
    out = np.empty((qa.shape[0], dbT.shape[1]), dtype=np.float64)
    for r0 in range(0, qa.shape[0], panel):
        out[r0:r0 + panel] = np.matmul(dequantize(qa[r0:r0 + panel], sa[r0:r0 + panel]), dbT)
    return out


def gemm_tn_abs(qa, sa, qb, sb, rows=None, cols=None) -> np.ndarray:
    """sum_k |dq(A)[m,k] * dq(B)[n,k]| in float64 (size of the terms)."""
    if rows is not None:
        qa, sa = qa[rows], sa[rows]
    if cols is not None:
        qb, sb = qb[cols], sb[cols]
    return np.matmul(np.abs(dequantize(qa, sa)), np.abs(dequantize(qb, sb)).T)


def grouped_gemm_tn(qx, sx, qw, sw, offsets, rows=None, cols=None, panel=None) -> np.ndarray:
    """Ragged grouped TN GEMM: rows [off[g], off[g+1]) of X times W[g]^T.

    Rows that belong to no group are NaN (they must not be written).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    G = len(offsets) - 1
    M = qx.shape[0]
    N = qw.shape[1]
    rows = np.arange(M) if rows is None else np.asarray(rows)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    out = np.full((len(rows), len(cols)), np.nan)
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        sel = np.nonzero((rows >= lo) & (rows < hi))[0]
        if sel.size == 0:
            continue
        out[sel] = gemm_tn(qx, sx, qw[g], sw[g], rows=rows[sel], cols=cols, panel=panel)
    return out
