"""The C ABI allocates, synchronises and reads back nothing, so a whole
quantize -> GEMM chain can be captured in a HIP graph and replayed.  Every
replay is checked bit for bit against the same calls run eagerly on the same
inputs, with eager work and synchronisations between the replays.  Repeated
launches are also bitwise deterministic (no atomics decide a value: amax is an
order-free maximum, dbias a fixed-order two-stage sum)."""

import numpy as np
import pytest

import mxfp8_block_scaled_quantize_amd as mx
import workloads
from gpu_util import log, need_gpu, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

ROW, COL, DB = mx.MXFP8_ROWWISE, mx.MXFP8_COLWISE, mx.MXFP8_DBIAS
AMAX, PACKED = mx.MXFP8_AMAX, mx.MXFP8_PACKED_SCALES


class Chain:
    """Preallocated buffers of one chain: row+col+dbias+amax quantize of X and
    W into packed scales, dense GEMM X W^T, grouped GEMM of X's rows over two
    experts (W's two row halves), a dense wgrad-shaped GEMM of the transposed
    copies, the dense GEMM again with the GELU epilogue and with the SwiGLU
    epilogue (W's rows read as N/2 gate rows then N/2 up rows), and GELU and its
    backward fused into row+col quantizes of the GEMM output (the backward
    with dbias, taking that output as both gradient and activation input), and
    the grouped GEMM with a per-expert bias and the SwiGLU epilogue, and the
    dense GEMM with the GELU epilogue writing MXFP8 (codes + packed scales)."""

    def __init__(self, torch, T, N, K):
        self.T, self.N, self.K = T, N, K
        dev = "cuda"
        self.x = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
        self.w = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        self.out = {}
        for name, (R, C) in (("x", (T, K)), ("w", (N, K))):
            o = {"q": torch.empty((R, C), dtype=torch.uint8, device=dev),
                 "p": torch.empty((C // 128, R), dtype=torch.int32, device=dev),
                 "qT": torch.empty((C, R), dtype=torch.uint8, device=dev),
                 "pT": torch.empty((R // 128, C), dtype=torch.int32, device=dev),
                 "db": torch.empty((C,), dtype=torch.float32, device=dev),
                 "amax": torch.empty((1,), dtype=torch.float32, device=dev)}
            nws = mx.mxfp8_quantize_workspace_bytes(R, C, ROW | COL | DB)
            o["ws"], o["nws"] = torch.empty((nws,), dtype=torch.uint8, device=dev), nws
            self.out[name] = o
        half = N // 2
        self.offsets = to_dev(np.array([0, T // 2 + 32, T], dtype=np.int32))
        self.c = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        self.cg = torch.empty((T, half), dtype=torch.bfloat16, device=dev)
        self.cw = torch.empty((K, K), dtype=torch.bfloat16, device=dev)
        self.cgelu = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        self.cswi = torch.empty((T, N // 2), dtype=torch.bfloat16, device=dev)
        self.bias = to_dev_bf16(workloads.normal_bf16((2, N // 2), 5, std=1.0))   # a bias row per expert
        self.cbias = torch.empty((T, N // 4), dtype=torch.bfloat16, device=dev)
        self.qmx = torch.empty((T, N), dtype=torch.uint8, device=dev)
        self.pmx = torch.empty((N // 128, T), dtype=torch.int32, device=dev)
        for name in ("h", "dh"):
            o = {"q": torch.empty((T, N), dtype=torch.uint8, device=dev),
                 "p": torch.empty((N // 128, T), dtype=torch.int32, device=dev),
                 "qT": torch.empty((N, T), dtype=torch.uint8, device=dev),
                 "pT": torch.empty((T // 128, N), dtype=torch.int32, device=dev),
                 "db": torch.empty((N,), dtype=torch.float32, device=dev),
                 "amax": torch.empty((1,), dtype=torch.float32, device=dev)}
            nws = mx.mxfp8_quantize_workspace_bytes(T, N, ROW | COL | DB)
            o["ws"], o["nws"] = torch.empty((nws,), dtype=torch.uint8, device=dev), nws
            self.out[name] = o

    def run(self):
        T, N, K = self.T, self.N, self.K
        for name, src, R in (("x", self.x, T), ("w", self.w, N)):
            o = self.out[name]
            mx.mxfp8_quantize_ex(src, R, K, K, ROW | COL | DB | AMAX | PACKED, o["q"], o["p"], o["qT"], o["pT"],
                                 o["db"], o["amax"], None, None, o["ws"], o["nws"])
        x, w = self.out["x"], self.out["w"]
        mx.mxfp8_gemm_ex(x["q"], x["p"], w["q"], w["p"], self.c, N, T, N, K, 0)
        mx.mxfp8_grouped_gemm_ex(x["q"], x["p"], w["q"], w["p"], self.offsets, 2, self.cg, N // 2, T, N // 2, K,
                                 mx.MXFP8_GEMM_SQRELU)
        # wgrad-shaped: [K x T] x [K x T]^T, reduction over the T tokens
        mx.mxfp8_gemm_ex(x["qT"], x["pT"], x["qT"], x["pT"], self.cw, K, K, K, T, 0)
        mx.mxfp8_gemm_ex(x["q"], x["p"], w["q"], w["p"], self.cgelu, N, T, N, K, mx.MXFP8_GEMM_GELU)
        mx.mxfp8_gemm_ex(x["q"], x["p"], w["q"], w["p"], self.cswi, N // 2, T, N // 2, K, mx.MXFP8_GEMM_SWIGLU)
        # W's N rows as two experts of N/2 rows, each N/4 gate rows then N/4 up rows, with their own bias rows
        mx.mxfp8_grouped_gemm_bias(x["q"], x["p"], w["q"], w["p"], self.offsets, 2, self.bias, self.cbias, N // 4,
                                   T, N // 4, K, mx.MXFP8_GEMM_SWIGLU)
        mx.mxfp8_gemm_mxfp8_out(x["q"], x["p"], w["q"], w["p"], None, self.qmx, N, self.pmx, T, N, K,
                                mx.MXFP8_GEMM_GELU)
        h, dh = self.out["h"], self.out["dh"]
        mx.mxfp8_quantize_ex(self.c, T, N, N, ROW | COL | AMAX | PACKED | mx.MXFP8_ACT_GELU, h["q"], h["p"],
                             h["qT"], h["pT"], None, h["amax"], None, None, None, 0)
        mx.mxfp8_quantize_ex(self.c, T, N, N, ROW | COL | DB | PACKED | mx.MXFP8_DACT_GELU, dh["q"], dh["p"],
                             dh["qT"], dh["pT"], dh["db"], None, None, self.c, dh["ws"], dh["nws"])

    def snapshot(self):
        snap = {"c": self.c.clone(), "cg": self.cg.clone(), "cw": self.cw.clone(), "cgelu": self.cgelu.clone(),
                "cswi": self.cswi.clone(), "cbias": self.cbias.clone(), "qmx": self.qmx.clone(),
                "pmx": self.pmx.clone()}
        for name, o in self.out.items():
            for k in ("q", "p", "qT", "pT", "db", "amax"):
                if not (name == "h" and k == "db") and not (name == "dh" and k == "amax"):
                    snap[name + "." + k] = o[k].clone()
        return snap


def assert_same(torch, got, ref, label):
    for k in ref:
        a, b = got[k], ref[k]
        if a.dtype in (torch.bfloat16, torch.float32):
            a, b = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32), \
                b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
        assert torch.equal(a, b), "%s: %s differs" % (label, k)


def inputs(torch, T, N, K, seed):
    x = to_dev_bf16(workloads.normal_bf16((T, K), seed))
    w = to_dev_bf16(workloads.normal_bf16((N, K), seed + 1, std=0.05))
    return x, w


def test_repeated_launches_are_bitwise_identical():
    torch = need_gpu()
    T, N, K = 768, 512, 640
    ch = Chain(torch, T, N, K)
    x, w = inputs(torch, T, N, K, 61)
    ch.x.copy_(x)
    ch.w.copy_(w)
    log("chain determinism T=%d N=%d K=%d" % (T, N, K))
    ch.run()
    torch.cuda.synchronize()
    first = ch.snapshot()
    for _ in range(3):
        ch.run()
        torch.cuda.synchronize()
        assert_same(torch, ch.snapshot(), first, "repeat")


def test_graph_replay_matches_eager():
    torch = need_gpu()
    T, N, K = 768, 512, 640
    ch = Chain(torch, T, N, K)
    x0, w0 = inputs(torch, T, N, K, 71)
    ch.x.copy_(x0)
    ch.w.copy_(w0)
    ch.run()                      # eager first: one-time per-device set-up happens outside the capture
    torch.cuda.synchronize()
    log("capture chain T=%d N=%d K=%d" % (T, N, K))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            ch.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        x, w = inputs(torch, T, N, K, 100 + 2 * rep)
        # eager reference on these inputs
        ch.x.copy_(x)
        ch.w.copy_(w)
        ch.run()
        torch.cuda.synchronize()
        ref = ch.snapshot()
        # poison every output, then replay the graph on the same inputs
        for o in ch.out.values():
            for k in ("q", "qT"):
                o[k].fill_(0xA5)
            for k in ("p", "pT"):
                o[k].fill_(-1)
            o["db"].fill_(-3.0)
            o["amax"].fill_(-7.0)
        for t in (ch.c, ch.cg, ch.cw, ch.cgelu, ch.cswi, ch.cbias):
            t.fill_(float("nan"))
        ch.qmx.fill_(0xA5)
        ch.pmx.fill_(-1)
        torch.cuda.synchronize()
        log("replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        assert_same(torch, ch.snapshot(), ref, "replay %d" % rep)
