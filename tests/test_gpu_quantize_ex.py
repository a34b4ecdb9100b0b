"""GPU parity of mxfp8_quantize_ex's fused extras against the oracle: scales
written directly in the packed word layout (bit-exact against the oracle's
packing of its own scales, and usable by the GEMM without a packing launch),
the per-tensor amax (exact) and the device-side noop flag (nothing written,
dbias and amax included)."""

import numpy as np
import pytest

import mxfp8_block_scaled_quantize_amd as mx
import oracle
import workloads
from gpu_util import log, need_gpu, to_dev, to_dev_bf16, to_host

pytestmark = pytest.mark.gpu

ROW, COL, DB = mx.MXFP8_ROWWISE, mx.MXFP8_COLWISE, mx.MXFP8_DBIAS
AMAX, PACKED = mx.MXFP8_AMAX, mx.MXFP8_PACKED_SCALES


def run_ex(bits, flags, noop_value=None, ld=None, act_bits=None):
    """mxfp8_quantize_ex into canary-filled buffers; returns host arrays.
    act_bits: the activation input for MXFP8_DACT_SQRELU (same shape)."""
    torch = need_gpu()
    R, C = bits.shape
    ld = C if ld is None else ld
    src = np.zeros((R, ld), dtype=np.uint16)
    src[:, :C] = bits
    x = to_dev_bf16(src)
    out = {}
    if flags & ROW:
        out["q_row"] = torch.full((R, C), 0xA5, dtype=torch.uint8, device="cuda")
        out["s_row"] = (torch.full((C // 128, R), -1, dtype=torch.int32, device="cuda") if flags & PACKED
                        else torch.full((R, C // 32), 0xA5, dtype=torch.uint8, device="cuda"))
    if flags & COL:
        out["q_colT"] = torch.full((C, R), 0xA5, dtype=torch.uint8, device="cuda")
        out["s_colT"] = (torch.full((R // 128, C), -1, dtype=torch.int32, device="cuda") if flags & PACKED
                         else torch.full((C, R // 32), 0xA5, dtype=torch.uint8, device="cuda"))
    if flags & DB:
        out["dbias"] = torch.full((C,), -5.0, dtype=torch.float32, device="cuda")
    if flags & AMAX:
        out["amax"] = torch.full((1,), -7.0, dtype=torch.float32, device="cuda")
    noop = None if noop_value is None else to_dev(np.array([noop_value], dtype=np.int32))
    act_in = None
    if act_bits is not None:
        asrc = np.zeros((R, ld), dtype=np.uint16)
        asrc[:, :C] = act_bits
        act_in = to_dev_bf16(asrc)
    nws = mx.mxfp8_quantize_workspace_bytes(R, C, flags)
    ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device="cuda")
    mx.mxfp8_quantize_ex(x, R, C, ld, flags, out.get("q_row"), out.get("s_row"), out.get("q_colT"),
                         out.get("s_colT"), out.get("dbias"), out.get("amax"), noop, act_in,
                         ws if nws else None, nws)
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in out.items()}


SHAPES = [(128, 128), (256, 384), (384, 1024), (640, 256), (1152, 640)]


@pytest.mark.parametrize("R,C", SHAPES)
@pytest.mark.parametrize("flags", [ROW, COL, ROW | COL, ROW | COL | DB, COL | DB])
def test_packed_scales_bit_exact(R, C, flags):
    bits = workloads.wide_range_bf16((R, C), R * 7 + C + flags, n_maxbf16=4, n_subnormal=64, n_subnormal_blocks=2)
    log("packed R=%d C=%d flags=%d" % (R, C, flags))
    got = run_ex(bits, flags | PACKED)
    if flags & ROW:
        q, s = oracle.quantize_rowwise(bits)
        assert np.array_equal(got["q_row"], q)
        assert np.array_equal(got["s_row"], oracle.pack_scales(s))
    if flags & COL:
        qT, sT = oracle.quantize_colwise(bits)
        assert np.array_equal(got["q_colT"], qT)
        assert np.array_equal(got["s_colT"], oracle.pack_scales(sT))


def test_packed_rowwise_with_ragged_rows_and_stride():
    bits = workloads.normal_bf16((200, 512), 3)      # rows need not be a multiple of 32 rowwise
    got = run_ex(bits, ROW | PACKED, ld=520)
    q, s = oracle.quantize_rowwise(bits)
    assert np.array_equal(got["q_row"], q)
    assert np.array_equal(got["s_row"], oracle.pack_scales(s))


def test_gemm_on_quantizer_packed_scales_matches_pack_kernel():
    torch = need_gpu()
    a = workloads.normal_bf16((384, 512), 11)
    b = workloads.normal_bf16((256, 512), 12, std=0.1)
    xa, xb = to_dev_bf16(a), to_dev_bf16(b)
    pa = mx.quantize(xa, packed=True)
    pb = mx.quantize(xb, packed=True)
    c1 = mx.gemm(pa["q_row"], pa["p_row"], pb["q_row"], pb["p_row"])
    ra, rb = mx.quantize(xa), mx.quantize(xb)
    c2 = mx.gemm(ra["q_row"], mx.pack_scales(ra["s_row"]), rb["q_row"], mx.pack_scales(rb["s_row"]))
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


@pytest.mark.parametrize("flags,R,C,ld", [(ROW, 512, 1024, None), (ROW, 300, 96, 104), (ROW | DB, 256, 256, None),
                                         (COL, 320, 192, None), (ROW | COL, 256, 384, None),
                                         (ROW | COL | DB, 128, 128, None), (ROW | PACKED, 256, 256, None)])
def test_amax_exact_on_every_path(flags, R, C, ld):
    bits = workloads.wide_range_bf16((R, C), R + C + flags, n_maxbf16=0, n_subnormal=8, n_subnormal_blocks=1)
    got = run_ex(bits, flags | AMAX, ld=ld)
    assert float(got["amax"][0]) == oracle.amax(bits)


def test_amax_special_values():
    z = np.zeros((256, 256), dtype=np.uint16)
    assert float(run_ex(z, ROW | AMAX)["amax"][0]) == 0.0            # all zero
    z[255, 255] = 0xC2F6                                              # -123 in the very last element
    assert float(run_ex(z, ROW | COL | AMAX)["amax"][0]) == 123.0
    z[0, 0] = workloads.BF16_MAX_BITS
    assert float(run_ex(z, COL | AMAX)["amax"][0]) == oracle.amax(z)


def test_amax_of_empty_tensor_is_zero():
    got = run_ex(np.zeros((0, 64), dtype=np.uint16), ROW | AMAX)
    assert float(got["amax"][0]) == 0.0


@pytest.mark.parametrize("flags", [ROW, ROW | COL | DB, COL | DB, ROW | PACKED, ROW | COL | PACKED])
def test_noop_flag_writes_nothing(flags):
    bits = workloads.normal_bf16((256, 256), 9)
    got = run_ex(bits, flags | AMAX, noop_value=1)
    for k, v in got.items():
        if v.dtype == np.uint8:
            assert np.all(v == 0xA5), k
        elif v.dtype == np.uint32:
            assert np.all(v == 0xFFFFFFFF), k
        elif k == "dbias":
            assert np.all(v == -5.0), k
        else:
            assert np.all(v == -7.0), k
    run = run_ex(bits, flags | AMAX, noop_value=0)                   # flag clear: normal results
    q, s = oracle.quantize_rowwise(bits)
    if flags & ROW:
        assert np.array_equal(run["q_row"], q)
    assert float(run["amax"][0]) == oracle.amax(bits)
    if flags & DB:
        assert np.allclose(run["dbias"], oracle.dbias(bits), rtol=1e-5, atol=1e-5)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["X", "W"])
def test_full_dense_packed_rowwise(name):
    """The default benchmark's quantize launches at full size: codes and packed
    scale words bit-exact, amax exact."""
    bits = workloads.dense_linear()[name]
    log("packed full %s %s" % (name, bits.shape))
    got = run_ex(bits, ROW | PACKED | AMAX)
    q, s = oracle.quantize_rowwise(bits)
    assert np.array_equal(got["q_row"], q)
    assert np.array_equal(got["s_row"], oracle.pack_scales(s))
    assert float(got["amax"][0]) == oracle.amax(bits)


@pytest.mark.slow
def test_full_stress_row_col_packed():
    """The stress step's row+col launch with packed scales (32768 x 8192, wide range)."""
    bits = workloads.stress()["A"]
    got = run_ex(bits, ROW | COL | PACKED)
    q, s = oracle.quantize_rowwise(bits)
    assert np.array_equal(got["q_row"], q)
    assert np.array_equal(got["s_row"], oracle.pack_scales(s))
    qT, sT = oracle.quantize_colwise(bits)
    assert np.array_equal(got["q_colT"], qT)
    assert np.array_equal(got["s_colT"], oracle.pack_scales(sT))


@pytest.mark.slow
def test_full_backward_packed():
    """The backward step's launches as timed: dY [16384 x 4096] (heavy tails,
    1 % zero blocks) row+col+dbias and X [16384 x 4096] columnwise, both
    writing packed scale words; codes and words bit-exact, dbias within the
    fp32 summation bound."""
    from test_gpu_quantize import check_dbias
    d = workloads.backward()
    log("backward dY row+col+dbias packed")
    got = run_ex(d["dY"], ROW | COL | DB | PACKED)
    q, s = oracle.quantize_rowwise(d["dY"])
    assert np.array_equal(got["q_row"], q)
    assert np.array_equal(got["s_row"], oracle.pack_scales(s))
    qT, sT = oracle.quantize_colwise(d["dY"])
    assert np.array_equal(got["q_colT"], qT)
    assert np.array_equal(got["s_colT"], oracle.pack_scales(sT))
    check_dbias(d["dY"], got["dbias"], "backward dY packed")
    log("backward X col packed")
    got = run_ex(d["X"], COL | PACKED)
    qT, sT = oracle.quantize_colwise(d["X"])
    assert np.array_equal(got["q_colT"], qT)
    assert np.array_equal(got["s_colT"], oracle.pack_scales(sT))


# ------------------------------------------------ activation-fused quantize

ACT, DACT = mx.MXFP8_ACT_SQRELU, mx.MXFP8_DACT_SQRELU


def act_inputs(R, C, seed):
    """Gradient-like x and activation input a whose products stay inside
    fp32's normal range: block magnitudes 2^-30 .. 2^30, no BF16 subnormals."""
    x = workloads.wide_range_bf16((R, C), seed, u_lo=-30, u_hi=30, n_maxbf16=0, n_subnormal=0, n_subnormal_blocks=0)
    a = workloads.wide_range_bf16((R, C), seed + 1, u_lo=-30, u_hi=30, n_maxbf16=0, n_subnormal=0,
                                  n_subnormal_blocks=0)
    return x, a


def check_act_result(got, v, flags, label):
    if flags & ROW:
        q, s = oracle.quantize_rowwise_values(v)
        assert np.array_equal(got["q_row"], q), label + " q_row"
        assert np.array_equal(got["s_row"], oracle.pack_scales(s) if flags & PACKED else s), label + " s_row"
    if flags & COL:
        qT, sT = oracle.quantize_colwise_values(v)
        assert np.array_equal(got["q_colT"], qT), label + " q_colT"
        assert np.array_equal(got["s_colT"], oracle.pack_scales(sT) if flags & PACKED else sT), label + " s_colT"
    if flags & DB:
        ref = oracle.dbias_values(v).astype(np.float64)
        mag = np.abs(v.astype(np.float64)).sum(axis=0)
        R = v.shape[0]
        depth = 8 + 2 + 3 + ((R + 127) // 128 + 7) // 8 + 3     # the fp32 addition chain of the kernel
        tol = 1.01 * depth * 2.0 ** -24 * mag + np.abs(ref) * 2.0 ** -24 + 2.0 ** -126
        err = np.abs(got["dbias"].astype(np.float64) - ref)
        assert np.all(err <= tol), "%s: dbias off by %g" % (label, err.max())
    if flags & AMAX:
        assert float(got["amax"][0]) == float(np.abs(v).max(initial=0.0)), label + " amax"


ACT_FLAGS = [ROW, COL, ROW | COL, ROW | DB, COL | DB, ROW | COL | DB, ROW | COL | AMAX, ROW | PACKED,
             ROW | COL | PACKED | DB]


@pytest.mark.parametrize("R,C", [(128, 128), (256, 384), (640, 256)])
@pytest.mark.parametrize("flags", ACT_FLAGS)
def test_sqrelu_quantize_bit_exact(R, C, flags):
    x, _ = act_inputs(R, C, 101 * R + C + flags)
    label = "sqrelu R=%d C=%d flags=%d" % (R, C, flags)
    log(label)
    got = run_ex(x, flags | ACT)
    check_act_result(got, oracle.act_sqrelu(x), flags, label)


@pytest.mark.parametrize("R,C", [(128, 128), (256, 384), (640, 256)])
@pytest.mark.parametrize("flags", ACT_FLAGS)
def test_dsqrelu_quantize_bit_exact(R, C, flags):
    g, a = act_inputs(R, C, 103 * R + C + flags)
    label = "dsqrelu R=%d C=%d flags=%d" % (R, C, flags)
    log(label)
    got = run_ex(g, flags | DACT, act_bits=a)
    check_act_result(got, oracle.dact_sqrelu(g, a), flags, label)


def test_activation_ragged_rows_and_stride():
    """Rowwise copies need no row multiple of 32; both inputs share ld_x."""
    g, a = act_inputs(200, 512, 7)
    got = run_ex(g, ROW | DB | AMAX | DACT, ld=520, act_bits=a)
    check_act_result(got, oracle.dact_sqrelu(g, a), ROW | DB | AMAX, "dsqrelu ragged")
    got = run_ex(g, ROW | AMAX | ACT, ld=520)
    check_act_result(got, oracle.act_sqrelu(g), ROW | AMAX, "sqrelu ragged")


def test_activation_special_values():
    """All-negative blocks (relu gives exact zeros: scale byte 0, codes 0), a
    zero activation input under a nonzero gradient, saturation at 448 * 2^X
    (a block whose largest square rounds up past the E4M3 range) and the
    amax of an all-zero result."""
    R, C = 128, 256
    x, a = act_inputs(R, C, 19)
    x[:32, :32] |= 0x8000                 # one all-negative 32 x 32 square
    a[32:64, :64] = 0                      # zero activation input
    x[64, 0:32] = workloads.f32_to_bf16_bits(np.full(32, 1.0, dtype=np.float32))
    x[64, 5] = 0x41F8                      # 31.0: 961 = 1.877 * 2^9, saturates to 448 * 2^1
    for flags in (ROW | COL | DB | AMAX, ROW | COL | PACKED):
        got = run_ex(x, flags | ACT)
        check_act_result(got, oracle.act_sqrelu(x), flags, "sqrelu special")
        got = run_ex(x, flags | DACT, act_bits=a)
        check_act_result(got, oracle.dact_sqrelu(x, a), flags, "dsqrelu special")
    neg = np.full((64, 64), 0xBF80, dtype=np.uint16)   # all -1.0
    got = run_ex(neg, ROW | COL | AMAX | ACT)
    assert float(got["amax"][0]) == 0.0
    assert not got["q_row"].any() and not got["s_row"].any() and not got["q_colT"].any()


@pytest.mark.parametrize("flags", [ROW | COL | DB | ACT, ROW | PACKED | DACT])
def test_activation_noop(flags):
    g, a = act_inputs(256, 256, 23)
    got = run_ex(g, flags | AMAX, noop_value=1, act_bits=a if flags & DACT else None)
    for k, v in got.items():
        if v.dtype == np.uint8:
            assert np.all(v == 0xA5), k
        elif v.dtype == np.uint32:
            assert np.all(v == 0xFFFFFFFF), k
        elif k == "dbias":
            assert np.all(v == -5.0), k
        else:
            assert np.all(v == -7.0), k


def test_dsqrelu_with_subnormal_activation_input():
    """Subnormal BF16 a under a large gradient gives normal products: 2 relu(a)
    must be exact for subnormal a too (a doubling that carries into the
    exponent field included)."""
    R, C = 128, 128
    rng = np.random.default_rng(29)
    a = rng.integers(1, 128, size=(R, C)).astype(np.uint16)          # positive subnormals
    a[:, ::3] |= 0x8000                                                # some negative ones (relu -> 0)
    a[::5, :] = 0x007F                                                 # largest subnormal: 2a is normal
    g = workloads.wide_range_bf16((R, C), 31, u_lo=100, u_hi=120, n_maxbf16=0, n_subnormal=0,
                                  n_subnormal_blocks=0)
    v = oracle.dact_sqrelu(g, a)
    assert np.all(np.abs(v[v != 0]) >= 2.0 ** -126)                   # inside the contract
    for flags in (ROW | COL | AMAX, ROW | COL | PACKED | DB):
        got = run_ex(g, flags | DACT, act_bits=a)
        check_act_result(got, v, flags, "dsqrelu subnormal a")


@pytest.mark.slow
def test_full_mlp_activation_quantize():
    """The MLP step's two activation launches at full size (8192 x 14336, row +
    col, packed scales): relu^2 of H, and the backward of dA through H with
    dbias.  Codes and scale words bit-exact, dbias within its bound, amax exact."""
    d = workloads.mlp_hidden()
    h, da = d["H"], d["dA"]
    log("full mlp relu^2 %s" % (h.shape,))
    got = run_ex(h, ROW | COL | PACKED | AMAX | ACT)
    check_act_result(got, oracle.act_sqrelu(h), ROW | COL | PACKED | AMAX, "full relu^2")
    del got
    log("full mlp dsqrelu %s" % (h.shape,))
    got = run_ex(da, ROW | COL | PACKED | DB | DACT, act_bits=h)
    check_act_result(got, oracle.dact_sqrelu(da, h), ROW | COL | PACKED | DB, "full dsqrelu")


@pytest.mark.slow
def test_full_square_and_linear_packed():
    """The dense step's square operands (rowwise, packed) and the linear
    step's dY [8192 x 14336] (row + col, packed) at full size, bit-exact."""
    sq = workloads.dense_square()
    for name in ("A", "B"):
        log("packed full square %s" % name)
        got = run_ex(sq[name], ROW | PACKED)
        q, s = oracle.quantize_rowwise(sq[name])
        assert np.array_equal(got["q_row"], q) and np.array_equal(got["s_row"], oracle.pack_scales(s)), name
        del got
    dy = workloads.normal_bf16((8192, 14336), 4)
    log("packed full linear dY row+col")
    got = run_ex(dy, ROW | COL | PACKED)
    q, s = oracle.quantize_rowwise(dy)
    assert np.array_equal(got["q_row"], q) and np.array_equal(got["s_row"], oracle.pack_scales(s))
    qT, sT = oracle.quantize_colwise(dy)
    assert np.array_equal(got["q_colT"], qT) and np.array_equal(got["s_colT"], oracle.pack_scales(sT))


@pytest.mark.slow
def test_full_moe_packed_rowwise():
    """The relu^2 MoE workload's operands, quantized into packed scales at full size."""
    data = workloads.moe()
    G, N, K = data["W"].shape
    for name, bits in (("X", data["X"]), ("W", data["W"].reshape(G * N, K))):
        log("packed full moe %s %s" % (name, bits.shape))
        got = run_ex(bits, ROW | PACKED)
        q, s = oracle.quantize_rowwise(bits)
        assert np.array_equal(got["q_row"], q) and np.array_equal(got["s_row"], oracle.pack_scales(s)), name
        del got


# ------------------------------------------------ GELU-fused quantize
#
# The kernel evaluates GELU and its derivative in fp32 with the device
# library's erfcf / expf, so its value w of an element is known only within
# a bound e of the exact value v (the oracle's float64 GELU).  The check below
# accepts exactly the outputs that some w in [v - e, v + e] (per element)
# would give: the block's scale byte between the bytes of the smallest and the
# largest possible block amax, each code between the codes of v - e and v + e
# under that byte.  Elements whose bound straddles a rounding boundary are
# counted; everywhere else the comparison is exact.

GELU, DGELU = mx.MXFP8_ACT_GELU, mx.MXFP8_DACT_GELU
ULP32 = 2.0 ** -24


def gelu_bound(x_bits):
    """|w - GELU(x)| <= (8 + 3 x^2) 2^-24 |GELU(x)|: twice the largest error
    measured over every BF16 input of the kernel's fp32 GELU.  For |x| >= 16
    the kernel's Phi(-|x|) is exactly 0 (exp(-128) underflows), so w is x or
    -0: within one rounding of the exact value."""
    x = oracle.bf16_value(x_bits)
    g = np.abs(oracle.gelu_f64(x))
    return np.where(np.abs(x) >= 16.0, ULP32 * g, (8.0 + 3.0 * x * x) * ULP32 * g)


def dgelu_bound(g_bits, a_bits):
    """|w - g GELU'(a)| <= |g| 8 2^-24 (|Phi(a)| + |a phi(a)|) + 2^-23 |v|:
    the derivative's sum within 8 ulp of its terms' magnitudes (measured: 3.6),
    then the product's rounding."""
    g = oracle.bf16_value(g_bits)
    t1, t2 = oracle.dgelu_terms(oracle.bf16_value(a_bits))
    return np.abs(g) * 8.0 * ULP32 * (np.abs(t1) + np.abs(t2)) + 2.0 * ULP32 * np.abs(g * (t1 + t2))


def unpack_words(p, dim):
    """Packed scale words uint32 [k/128][dim] -> bytes [dim][k/32], checked
    to be the oracle's packing of the bytes returned."""
    w = np.ascontiguousarray(p).view(np.uint32)
    T = w.shape[0]
    s = np.ascontiguousarray(w.view(np.uint8).reshape(T, dim, 4).transpose(1, 0, 2).reshape(dim, 4 * T))
    assert np.array_equal(oracle.pack_scales(s), w)
    return s


def check_bounded_copy(q, s, v, e, label):
    """Codes q [n][m] and scale bytes s [n][m/32] (blocks of 32 along m) of
    values within v +- e.  Returns the numbers of codes and of blocks that
    the bound leaves open (values on an E4M3 rounding tie or a block amax on
    a power of two, mostly where GELU(x) is x to within 1e-9)."""
    n, m = v.shape
    av = np.abs(v).reshape(n, m // 32, 32)
    ae = e.reshape(n, m // 32, 32)
    b_lo = oracle.scale_bytes(np.maximum(av - ae, 0.0).max(axis=2))
    b_hi = oracle.scale_bytes((av + ae).max(axis=2))
    bad = (s < b_lo) | (s > b_hi)
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError("%s: %d scale bytes outside their bound, first (%d,%d) got %d want [%d,%d]" % (
            label, bad.sum(), i, j, s[i, j], b_lo[i, j], b_hi[i, j]))
    X = np.repeat(oracle.e8m0_decode(s), 32, axis=1)
    d = oracle.e4m3_decode(q)
    assert not np.isnan(d).any(), label + ": NaN code"
    d_lo = oracle.e4m3_decode(oracle.e4m3_encode((v - e) / X))
    d_hi = oracle.e4m3_decode(oracle.e4m3_encode((v + e) / X))
    bad = (d < d_lo) | (d > d_hi)
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError("%s: %d codes outside their bound, first (%d,%d) v=%g e=%g got %g want [%g,%g]" % (
            label, bad.sum(), i, j, v[i, j], e[i, j], d[i, j], d_lo[i, j], d_hi[i, j]))
    return int(np.sum(d_lo != d_hi)), int(np.sum(b_lo != b_hi))


def check_open(f, v, label, max_open=0.02):
    """At most 2 % of the codes and of the blocks open (plus 2 codes and one
    block, for tiny tensors)."""
    n = v.size
    assert f[0] <= max_open * n + 2 and f[1] <= max_open * n / 32 + 1, \
        "%s: open (codes, blocks) %s of (%d, %d)" % (label, f, n, n // 32)


def check_gelu_result(got, v, e, flags, label):
    R, C = v.shape
    if flags & ROW:
        s = unpack_words(got["s_row"], R) if flags & PACKED else got["s_row"]
        check_open(check_bounded_copy(got["q_row"], s, v, e, label + " row"), v, label + " row")
    if flags & COL:
        s = unpack_words(got["s_colT"], C) if flags & PACKED else got["s_colT"]
        f = check_bounded_copy(got["q_colT"], s, np.ascontiguousarray(v.T), np.ascontiguousarray(e.T),
                               label + " col")
        check_open(f, v, label + " col")
    if flags & DB:
        ref = v.sum(axis=0)
        mag = np.abs(v).sum(axis=0)
        depth = 8 + 2 + 3 + ((R + 127) // 128 + 7) // 8 + 3     # the fp32 addition chain of the kernel
        tol = 1.01 * depth * ULP32 * (mag + e.sum(axis=0)) + e.sum(axis=0) + np.abs(ref) * ULP32 + 2.0 ** -126
        err = np.abs(got["dbias"].astype(np.float64) - ref)
        assert np.all(err <= tol), "%s: dbias off by %g" % (label, (err - tol).max())
    if flags & AMAX:
        a = float(got["amax"][0])
        lo = float(np.maximum(np.abs(v) - e, 0.0).max(initial=0.0))
        hi = float((np.abs(v) + e).max(initial=0.0))
        assert lo <= a <= hi, "%s: amax %r outside [%r, %r]" % (label, a, lo, hi)


def gelu_case(R, C, seed):
    x = workloads.preact_bf16((R, C), seed)
    return x, oracle.act_gelu(x), gelu_bound(x)


def dgelu_case(R, C, seed):
    g = workloads.wide_range_bf16((R, C), seed, u_lo=-30, u_hi=30, n_maxbf16=0, n_subnormal=0,
                                  n_subnormal_blocks=0)
    a = workloads.preact_bf16((R, C), seed + 1, floor=-10.0)
    return g, a, oracle.dact_gelu(g, a), dgelu_bound(g, a)


def test_gelu_bounds_cover_the_contract():
    """The inputs stay where the fp32 results are normal numbers (the
    contract), and the bounds are far below an E4M3 step (2^-4 relative)."""
    x, v, e = gelu_case(256, 384, 1)
    assert np.all((np.abs(v) >= 2.0 ** -126) | (v == 0)) and np.all(e <= 2.0 ** -10 * np.abs(v))
    g, a, v, e = dgelu_case(256, 384, 2)
    nz = v != 0
    assert np.all(np.abs(v[nz]) >= 2.0 ** -126)


@pytest.mark.parametrize("R,C", [(128, 128), (256, 384), (640, 256)])
@pytest.mark.parametrize("flags", ACT_FLAGS)
def test_gelu_quantize(R, C, flags):
    x, v, e = gelu_case(R, C, 107 * R + C + flags)
    label = "gelu R=%d C=%d flags=%d" % (R, C, flags)
    log(label)
    got = run_ex(x, flags | GELU)
    check_gelu_result(got, v, e, flags, label)


@pytest.mark.parametrize("R,C", [(128, 128), (256, 384), (640, 256)])
@pytest.mark.parametrize("flags", ACT_FLAGS)
def test_dgelu_quantize(R, C, flags):
    g, a, v, e = dgelu_case(R, C, 109 * R + C + flags)
    label = "dgelu R=%d C=%d flags=%d" % (R, C, flags)
    log(label)
    got = run_ex(g, flags | DGELU, act_bits=a)
    check_gelu_result(got, v, e, flags, label)


def test_gelu_ragged_rows_and_stride():
    g, a, v, e = dgelu_case(200, 512, 11)
    log("dgelu ragged")
    got = run_ex(g, ROW | DB | AMAX | DGELU, ld=520, act_bits=a)
    check_gelu_result(got, v, e, ROW | DB | AMAX, "dgelu ragged")
    x, v, e = gelu_case(200, 512, 13)
    log("gelu ragged")
    got = run_ex(x, ROW | AMAX | GELU, ld=520)
    check_gelu_result(got, v, e, ROW | AMAX, "gelu ragged")


def test_gelu_special_values():
    """Zero blocks (GELU(0) = 0: byte 0, codes 0), blocks far on the positive
    side (GELU(x) = x to within 1e-15: the scale bytes of x itself),
    saturation (GELU(31) = 31 = 1.9375 * 2^4 rounds past 448 * 2^-4), a zero
    activation input under a nonzero gradient (GELU'(0) = 1/2), and blocks
    of huge inputs (20 .. 3e38: GELU(x) = x and GELU'(a) = 1 exactly, their
    negatives give zeros)."""
    R, C = 128, 256
    x = workloads.preact_bf16((R, C), 17)
    x[:32, :32] = 0
    x[32:64, 32:64] = workloads.f32_to_bf16_bits(np.linspace(8.0, 30.0, 1024, dtype=np.float32).reshape(32, 32))
    x[64, 0:32] = workloads.f32_to_bf16_bits(np.full(32, 1.0, dtype=np.float32))
    x[64, 5] = 0x41F8                      # 31.0
    huge = workloads.f32_to_bf16_bits(np.geomspace(20.0, 3.0e38, 32).astype(np.float32))
    x[96, 64:96] = huge                    # GELU(x) = x
    x[97, 64:96] = huge | 0x8000           # GELU(x) = -0 (the exact value underflows)
    v, e = oracle.act_gelu(x), gelu_bound(x)
    for flags in (ROW | COL | DB | AMAX, ROW | COL | PACKED):
        log("gelu special flags=%d" % flags)
        got = run_ex(x, flags | GELU)
        check_gelu_result(got, v, e, flags, "gelu special")
        if not flags & PACKED:
            assert not got["q_row"][:32, :32].any() and not got["s_row"][:32, :1].any()
            _, s = oracle.quantize_rowwise(x[32:64, 32:64])          # block amax 30: far from a power of 2
            assert np.array_equal(got["s_row"][32:64, 1:2], s)
            assert got["q_row"][64, 5] == 0x7E and got["s_row"][64, 0] == 127 - 4
            q, s = oracle.quantize_rowwise(huge[None, :])
            assert np.array_equal(got["q_row"][96, 64:96], q[0]) and got["s_row"][96, 2] == s[0, 0]
            assert got["s_row"][97, 2] == 0 and np.all(got["q_row"][97, 64:96] & 0x7F == 0)
    g = workloads.wide_range_bf16((R, C), 19, u_lo=-10, u_hi=10, n_maxbf16=0, n_subnormal=0, n_subnormal_blocks=0)
    a = workloads.preact_bf16((R, C), 21, floor=-10.0)
    a[32:64, :64] = 0
    a[96, 64:96] = huge                    # GELU'(a) = 1: v = g
    a[97, 64:96] = huge | 0x8000           # GELU'(a) = 0
    v, e = oracle.dact_gelu(g, a), dgelu_bound(g, a)
    for flags in (ROW | COL | DB | AMAX, ROW | COL | PACKED):
        log("dgelu special flags=%d" % flags)
        got = run_ex(g, flags | DGELU, act_bits=a)
        check_gelu_result(got, v, e, flags, "dgelu special")
        if not flags & PACKED:
            q, s = oracle.quantize_rowwise_values(v[32:64, :64])   # g / 2 is exact
            assert np.array_equal(got["q_row"][32:64, :64], q) and np.array_equal(got["s_row"][32:64, :2], s)
            q, s = oracle.quantize_rowwise(g[96:97, 64:96])
            assert np.array_equal(got["q_row"][96, 64:96], q[0]) and got["s_row"][96, 2] == s[0, 0]
            assert got["s_row"][97, 2] == 0 and np.all(got["q_row"][97, 64:96] & 0x7F == 0)


@pytest.mark.parametrize("flags", [ROW | COL | DB | GELU, ROW | PACKED | DGELU])
def test_gelu_noop(flags):
    g, a, _, _ = dgelu_case(256, 256, 23)
    got = run_ex(g, flags | AMAX, noop_value=1, act_bits=a if flags & DGELU else None)
    for k, v in got.items():
        if v.dtype == np.uint8:
            assert np.all(v == 0xA5), k
        elif v.dtype == np.uint32:
            assert np.all(v == 0xFFFFFFFF), k
        elif k == "dbias":
            assert np.all(v == -5.0), k
        else:
            assert np.all(v == -7.0), k


@pytest.mark.slow
def test_full_mlp_gelu_quantize():
    """A GELU MLP's two activation launches at full size (8192 x 14336, row +
    col, packed scales): GELU of H (amax), and the backward of dA through H
    with dbias."""
    d = workloads.mlp_hidden()
    h, da = d["H"], d["dA"]
    log("full mlp gelu %s" % (h.shape,))
    got = run_ex(h, ROW | COL | PACKED | AMAX | GELU)
    check_gelu_result(got, oracle.act_gelu(h), gelu_bound(h), ROW | COL | PACKED | AMAX, "full gelu")
    del got
    log("full mlp dgelu %s" % (h.shape,))
    got = run_ex(da, ROW | COL | PACKED | DB | DGELU, act_bits=h)
    check_gelu_result(got, oracle.dact_gelu(da, h), dgelu_bound(da, h), ROW | COL | PACKED | DB, "full dgelu")
