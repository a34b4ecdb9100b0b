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


def run_ex(bits, flags, noop_value=None, ld=None):
    """mxfp8_quantize_ex into canary-filled buffers; returns host arrays."""
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
    nws = mx.mxfp8_quantize_workspace_bytes(R, C, flags)
    ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device="cuda")
    mx.mxfp8_quantize_ex(x, R, C, ld, flags, out.get("q_row"), out.get("s_row"), out.get("q_colT"),
                         out.get("s_colT"), out.get("dbias"), out.get("amax"), noop, ws if nws else None, nws)
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
