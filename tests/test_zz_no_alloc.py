"""The allocation-free quantize entry point (mxfp8_quantize_ex_noalloc: dbias
partial sums in the library's static device scratch) against mxfp8_quantize_ex
with a caller workspace, through the C ABI: two calls in a row, the second on
a smaller input, every output byte equal (same kernels, same summation order),
and dbias within its bound of the oracle."""

import ctypes

import numpy as np
import pytest

import mxfp8_block_scaled_quantize_amd as mx
import oracle
import workloads
from gpu_util import log, need_gpu, to_dev_bf16, to_host

pytestmark = pytest.mark.gpu

FLAGS = (mx.MXFP8_ROWWISE | mx.MXFP8_COLWISE | mx.MXFP8_DBIAS | mx.MXFP8_AMAX | mx.MXFP8_PACKED_SCALES)


def _outputs(torch, R, C):
    dev = "cuda"
    return {"q": torch.full((R, C), 0x5A, dtype=torch.uint8, device=dev),
            "p": torch.full((C // 128, R), 7, dtype=torch.int32, device=dev),
            "qT": torch.full((C, R), 0x5A, dtype=torch.uint8, device=dev),
            "pT": torch.full((R // 128, C), 7, dtype=torch.int32, device=dev),
            "db": torch.full((C,), -1.0, dtype=torch.float32, device=dev),
            "am": torch.full((1,), -1.0, dtype=torch.float32, device=dev)}


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _run(torch, L, x, R, C, noalloc):
    o = _outputs(torch, R, C)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        rc = L.mxfp8_quantize_ex_noalloc(_p(x), R, C, C, FLAGS, _p(o["q"]), _p(o["p"]), _p(o["qT"]), _p(o["pT"]),
                                         _p(o["db"]), _p(o["am"]), None, None, st)
    else:
        nws = L.mxfp8_quantize_workspace_bytes(R, C, FLAGS)
        ws = torch.empty((nws,), dtype=torch.uint8, device="cuda")
        o["ws"] = ws
        rc = L.mxfp8_quantize_ex(_p(x), R, C, C, FLAGS, _p(o["q"]), _p(o["p"]), _p(o["qT"]), _p(o["pT"]),
                                 _p(o["db"]), _p(o["am"]), None, None, _p(ws), nws, st)
    assert rc == 0, mx.mxfp8_status_string(rc)
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in o.items() if k != "ws"}


def test_noalloc_quantize_matches_the_workspace_entry_point():
    torch = need_gpu()
    L = mx.lib()
    for R, C, seed in ((1024, 896, 61), (384, 256, 62)):      # the second call is smaller
        bits = workloads.student_t_bf16((R, C), seed)
        x = to_dev_bf16(bits)
        log("noalloc quantize R=%d C=%d flags=%d" % (R, C, FLAGS))
        got = _run(torch, L, x, R, C, noalloc=True)
        want = _run(torch, L, x, R, C, noalloc=False)
        for k in want:
            assert np.array_equal(got[k].view(np.uint8), want[k].view(np.uint8)), (R, C, k)
        ref = oracle.dbias(bits)
        absum = np.abs(oracle.bf16_value(bits)).sum(axis=0)
        assert np.all(np.abs(got["db"].astype(np.float64) - ref) <= 1e-5 * absum + 1e-30), (R, C)
        assert got["am"][0] == np.float32(oracle.amax(bits))


def test_noalloc_quantize_rejects_requests_beyond_the_scratch():
    torch = need_gpu()
    L = mx.lib()
    R, C = 1025 * 128, 2048          # partial sums of 1025 row tiles x 2048 columns: 8 MiB + 8 KiB
    assert L.mxfp8_quantize_workspace_bytes(R, C, FLAGS) > mx.MXFP8_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((128, 128), dtype=torch.bfloat16, device="cuda")   # never read: rejected first
    with pytest.raises(mx.MXFP8Error, match="WORKSPACE"):
        mx.mxfp8_quantize_ex_noalloc(x, R, C, C, FLAGS, x, x, x, x, x, x)
