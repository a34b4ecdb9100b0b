"""Benchmark of the MXFP8 hot path on one MI355X.

Default workload (the one whose JSON line is the benchmark): the wide-range
stress configuration, the largest dense shape.  One step = rowwise +
columnwise MXFP8 quantize of A BF16[32768x8192] (32-element blocks scaled by
2^u, u uniform in [-40, 40], with max-BF16 and subnormal values injected) and
rowwise quantize of B BF16[8192x8192] (same recipe without max-BF16), each
writing its scales directly in the GEMM's packed word layout, then the TN
GEMM C[32768x8192] = A B^T (K = 8192) with BF16 output.  Inputs are resident
in HBM before timing starts.

``value`` is the end-to-end GEMM throughput of the step (GEMM FLOPs / wall
time of the whole step, quantize included).  ``roofline`` is the dominant
kernel (the GEMM) against the FP8 MFMA peak, timed with HIP events recorded on
its launch stream; ``quantize_roofline`` is the largest quantize launch (A
row+col, 1.09 GB) against the HBM peak; ``cpu_baseline`` is the CPU oracle
running whole steps of the same workload on the host.  Per-launch times are
reported as mean, median, min and max over the timed steps.

``--workload dense|backward|moe|moe_sqrelu|moe_swiglu|linear|mlp|mlp_gelu|mlp_fwd|moe_fwd`` measures the other
workloads the same way: rowwise quantize and the TN GEMMs 8192x14336x4096 and
8192^3; row+col+dbias quantize and the wgrad GEMM on the columnwise copies;
the ragged grouped MoE GEMM (also with the squared-ReLU or the SwiGLU
epilogue of an MoE first projection); one MXFP8 linear-layer training step (fprop, dgrad, wgrad
accumulated into a BF16 main gradient); one squared-ReLU (or GELU) MLP
training step (six GEMMs, the activation and its backward fused into the
quantize launches); the GELU MLP's inference forward (FC1 writing its GELU
output as MXFP8, FC2 reading it) and the MoE block's (the grouped first
projection writing its SwiGLU output as MXFP8 for the grouped second).  They are reporting aids next to the
default line.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP8 GEMM TFLOPS (% FP8 MFMA peak) + quantize GB/s (% HBM peak), 1 GPU"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0   # dense FP8 MFMA, MI355X published figure


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="stress",
                   choices=["stress", "dense", "backward", "moe", "moe_sqrelu", "moe_swiglu", "linear", "mlp",
                            "mlp_gelu", "mlp_fwd", "moe_fwd"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU-oracle time: whole oracle steps are repeated until reached "
                        "(at least one whole step runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one plain 256 MiB device copy (reference for HBM byte counters)")
    p.add_argument("--no-vendor-reference", action="store_true",
                   help="skip the reference run of PyTorch's MXFP8 GEMM (torch._scaled_mm with E8M0 block scales, "
                        "hipBLASLt on ROCm) on the dominant GEMM's shape, after the timed region")
    p.add_argument("--no-mfma-calibration", action="store_true",
                   help="skip the reference run of the scaled FP8 MFMA fed from registers only (libmxfp8_calib.so) "
                        "on the dominant GEMM's tile grid, as many launches as timed steps, after the timed region: "
                        "the rate a GEMM that still moves its operands could at most reach on this GPU at this power")
    return p.parse_args()


GEMM_SOURCES = ("mxfp8_block_scaled_quantize_amd/csrc/gemm.hip", "mxfp8_block_scaled_quantize_amd/csrc/mx_device.h")
QUANTIZE_SOURCES = ("mxfp8_block_scaled_quantize_amd/csrc/quantize.hip",
                    "mxfp8_block_scaled_quantize_amd/csrc/mx_device.h")


def source_hash(files=GEMM_SOURCES):
    """Hash of the sources that define a kernel (profile traffic is tied to it)."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def gemm_source_hash():
    return source_hash(GEMM_SOURCES)


def profiled_traffic(kernel_key, files=GEMM_SOURCES):
    """HBM-side bytes per launch from the rocprofv3 summaries in profiles/, or None
    when no summary was taken for the current sources of that kernel."""
    src = source_hash(files)
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    for name in sorted(os.listdir(pdir)):
        with open(os.path.join(pdir, name)) as fh:
            for line in fh:
                parts = line.split()
                if len(parts) >= 5 and parts[0] == "traffic" and parts[1] == kernel_key and parts[2] == "src=" + src:
                    kv = dict(p.split("=", 1) for p in parts[3:] if "=" in p)
                    return int(kv["read_bytes"]) + int(kv["write_bytes"]), name
    return None


def quant_bytes(rows, cols, copies, dbias=False, inputs=1):
    """Algorithmic bytes of a quantize: read 2 B per element and input (x, and
    the activation input of the fused backward activation), write 1 + 1/32 B
    per element and copy, plus 4 B per column for dbias."""
    return rows * cols * (2 * inputs + copies * (1 + 1.0 / 32)) + (4 * cols if dbias else 0)


class Op:
    """One launch of the step: kind (quantize / pack / gemm), label, callable
    taking the stream, algorithmic work (bytes for quantize / pack, FLOPs for
    gemm)."""

    def __init__(self, kind, label, fn, work):
        self.kind, self.label, self.fn, self.work = kind, label, fn, work


def build_ops(workload, dev):
    """Upload the workload's inputs, allocate outputs and return the step's launches."""
    import numpy as np
    import torch

    import mxfp8_block_scaled_quantize_amd as mx
    import workloads

    def upload(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    ops, keep = [], []

    def quantize_op(label, bits, flags, packed=False, act_in=None):
        """Quantize launch (+ one packing launch per copy, unless the quantizer
        writes the packed scale words itself).  bits: host BF16 bit patterns,
        or a device BF16 tensor written by an earlier launch of the step."""
        R, C = bits.shape
        b = {"x": bits if isinstance(bits, torch.Tensor) else upload(bits), "act_in": act_in}
        if flags & mx.MXFP8_ROWWISE:
            b["q"] = torch.empty((R, C), dtype=torch.uint8, device=dev)
            b["s"] = torch.empty((R, C // 32), dtype=torch.uint8, device=dev)
            b["p"] = torch.empty((C // 128, R), dtype=torch.int32, device=dev)
        if flags & mx.MXFP8_COLWISE:
            b["qT"] = torch.empty((C, R), dtype=torch.uint8, device=dev)
            b["sT"] = torch.empty((C, R // 32), dtype=torch.uint8, device=dev)
            b["pT"] = torch.empty((R // 128, C), dtype=torch.int32, device=dev)
        if flags & mx.MXFP8_DBIAS:
            b["db"] = torch.empty((C,), dtype=torch.float32, device=dev)
        nws = mx.mxfp8_quantize_workspace_bytes(R, C, flags)
        b["ws"] = torch.empty((max(nws, 16),), dtype=torch.uint8, device=dev) if nws else None
        keep.append(b)
        copies = int(bool(flags & mx.MXFP8_ROWWISE)) + int(bool(flags & mx.MXFP8_COLWISE))
        work = quant_bytes(R, C, copies, bool(flags & mx.MXFP8_DBIAS), 2 if act_in is not None else 1)
        if packed:
            ops.append(Op("quantize", label + " packed", lambda st: mx.mxfp8_quantize_ex(
                b["x"], R, C, C, flags | mx.MXFP8_PACKED_SCALES, b.get("q"), b.get("p"), b.get("qT"), b.get("pT"),
                b.get("db"), act_in=b["act_in"], workspace=b["ws"], workspace_bytes=nws, stream=st), work))
            return b
        ops.append(Op("quantize", label, lambda st: mx.mxfp8_quantize(
            b["x"], R, C, C, flags, b.get("q"), b.get("s"), b.get("qT"), b.get("sT"), b.get("db"),
            b["ws"], nws, stream=st), work))
        # packing reads the byte scales and writes the same bytes as words
        if flags & mx.MXFP8_ROWWISE:
            ops.append(Op("pack", label + " row", lambda st: mx.mxfp8_pack_scales(
                b["s"], R, C, C // 32, b["p"], stream=st), 2.0 * R * C / 32))
        if flags & mx.MXFP8_COLWISE:
            ops.append(Op("pack", label + " col", lambda st: mx.mxfp8_pack_scales(
                b["sT"], C, R, R // 32, b["pT"], stream=st), 2.0 * R * C / 32))
        return b

    def gemm_op(a, pa, b, pb, M, N, K, accumulate=False, name="", out=None):
        c = torch.zeros((M, N), dtype=torch.bfloat16, device=dev)
        keep.append(c)
        label = name + "%dx%dx%d" % (M, N, K)
        flags = mx.MXFP8_GEMM_ACCUMULATE if accumulate else 0
        ops.append(Op("gemm", label, lambda st: mx.mxfp8_gemm_ex(a, pa, b, pb, c, N, M, N, K, flags, stream=st),
                      2.0 * M * N * K))
        if out is not None:
            out.append(c)
        return label

    ROW, COL, DB = mx.MXFP8_ROWWISE, mx.MXFP8_COLWISE, mx.MXFP8_DBIAS
    host = {}
    if workload == "dense":
        lin, sq = workloads.dense_linear(), workloads.dense_square()
        host = {"X": lin["X"], "W": lin["W"], "A": sq["A"], "B": sq["B"]}
        # each GEMM right after the quantize launches that produce its operands
        bx = quantize_op("X[8192x4096]", lin["X"], ROW, packed=True)
        bw = quantize_op("W[14336x4096]", lin["W"], ROW, packed=True)
        dominant = gemm_op(bx["q"], bx["p"], bw["q"], bw["p"], 8192, 14336, 4096)
        ba = quantize_op("A[8192x8192]", sq["A"], ROW, packed=True)
        bb = quantize_op("B[8192x8192]", sq["B"], ROW, packed=True)
        gemm_op(ba["q"], ba["p"], bb["q"], bb["p"], 8192, 8192, 8192)
        desc = ("dense linear layer: rowwise MXFP8 quantize of X[8192x4096] and W[14336x4096] writing the packed "
                "scale words, TN GEMM 8192x14336x4096; the same for A[8192x8192], B[8192x8192] and the TN GEMM "
                "8192x8192x8192; BF16 out")
    elif workload == "backward":
        d = workloads.backward()
        host = d
        bd = quantize_op("dY[16384x4096] row+col+dbias", d["dY"], ROW | COL | DB, packed=True)
        bx = quantize_op("X[16384x4096] col", d["X"], COL, packed=True)
        dominant = gemm_op(bd["qT"], bd["pT"], bx["qT"], bx["pT"], 4096, 4096, 16384)
        desc = ("backward: dY[16384x4096] = 0.1*t(3) with 1% zero 32x32 tiles, rowwise+columnwise quantize with "
                "fused dbias; X[16384x4096] columnwise; both writing the packed scale words; wgrad TN GEMM "
                "4096x4096x16384 on the transposed copies")
    elif workload == "stress":
        d = workloads.stress()
        host = d
        ba = quantize_op("A[32768x8192] row+col", d["A"], ROW | COL, packed=True)
        bb = quantize_op("B[8192x8192]", d["B"], ROW, packed=True)
        dominant = gemm_op(ba["q"], ba["p"], bb["q"], bb["p"], 32768, 8192, 8192)
        desc = ("wide-range stress: A[32768x8192] (2^u block scales, max BF16, subnormals) rowwise+columnwise, "
                "B[8192x8192] rowwise, TN GEMM 32768x8192x8192")
    elif workload == "linear":
        lin = workloads.dense_linear()
        T, K = lin["X"].shape
        N = lin["W"].shape[0]
        dy = workloads.normal_bf16((T, N), 4)
        host = {"X": lin["X"], "W": lin["W"], "dY": dy}
        bx = quantize_op("X[%dx%d] row+col" % (T, K), lin["X"], ROW | COL, packed=True)
        bw = quantize_op("W[%dx%d] row+col" % (N, K), lin["W"], ROW | COL, packed=True)
        dominant = gemm_op(bx["q"], bx["p"], bw["q"], bw["p"], T, N, K, name="fprop ")
        bd = quantize_op("dY[%dx%d] row+col" % (T, N), dy, ROW | COL, packed=True)
        gemm_op(bd["q"], bd["p"], bw["qT"], bw["pT"], T, K, N, name="dgrad ")
        gemm_op(bd["qT"], bd["pT"], bx["qT"], bx["pT"], N, K, T, accumulate=True, name="wgrad+= ")
        desc = ("MXFP8 linear layer training step: X[%d x %d] N(0,1), W[%d x %d] N(0,0.02), dY N(0,1); "
                "row+col quantize of X, W, dY, fprop %dx%dx%d, dgrad %dx%dx%d on W's transposed copy, wgrad "
                "%dx%dx%d on the transposed copies accumulated into a BF16 main gradient"
                % (T, K, N, K, T, N, K, T, K, N, N, K, T))
    elif workload in ("mlp", "mlp_gelu"):
        lin = workloads.mlp()
        host = dict(lin, **workloads.mlp_hidden())
        T, D = lin["X"].shape
        F = lin["W1"].shape[0]
        w2, dy = lin["W2"], lin["dY"]
        gelu = workload == "mlp_gelu"
        ACT, DACT = ((mx.MXFP8_ACT_GELU, mx.MXFP8_DACT_GELU) if gelu
                     else (mx.MXFP8_ACT_SQRELU, mx.MXFP8_DACT_SQRELU))
        aname, dname, fname = (("GELU(H)", "dA*GELU'(H)", "GELU") if gelu else ("relu^2(H)", "dA*2relu(H)", "squared-ReLU"))
        h, da = [], []
        bx = quantize_op("X[%dx%d] row+col" % (T, D), lin["X"], ROW | COL, packed=True)
        bw1 = quantize_op("W1[%dx%d] row+col" % (F, D), lin["W1"], ROW | COL, packed=True)
        dominant = gemm_op(bx["q"], bx["p"], bw1["q"], bw1["p"], T, F, D, name="fc1 ", out=h)
        ba = quantize_op("%s[%dx%d] row+col" % (aname, T, F), h[0], ROW | COL | ACT, packed=True)
        bw2 = quantize_op("W2[%dx%d] row+col" % (D, F), w2, ROW | COL, packed=True)
        gemm_op(ba["q"], ba["p"], bw2["q"], bw2["p"], T, D, F, name="fc2 ")
        bdy = quantize_op("dY[%dx%d] row+col" % (T, D), dy, ROW | COL, packed=True)
        gemm_op(bdy["q"], bdy["p"], bw2["qT"], bw2["pT"], T, F, D, name="fc2 dgrad ", out=da)
        gemm_op(bdy["qT"], bdy["pT"], ba["qT"], ba["pT"], D, F, T, name="fc2 wgrad ")
        bdh = quantize_op("dH=%s[%dx%d] row+col+dbias" % (dname, T, F), da[0], ROW | COL | DB | DACT, packed=True,
                          act_in=h[0])
        gemm_op(bdh["q"], bdh["p"], bw1["qT"], bw1["pT"], T, D, F, name="fc1 dgrad ")
        gemm_op(bdh["qT"], bdh["pT"], bx["qT"], bx["pT"], F, D, T, name="fc1 wgrad ")
        desc = ("%s MLP training step, tokens %d, d_model %d, d_ff %d: X N(0,1), W1 N(0,0.02), "
                "W2 N(0,0.02), dY N(0,1); row+col quantize of X, W1, W2, dY; FC1 GEMM; the activation fused into "
                "the quantize of its BF16 output; FC2 GEMM; FC2 dgrad and wgrad; the activation's backward fused "
                "into the row+col+dbias quantize of FC2's dgrad output; FC1 dgrad and wgrad" % (fname, T, D, F))
    elif workload == "mlp_fwd":
        lin = workloads.mlp()
        host = lin
        T, D = lin["X"].shape
        F = lin["W1"].shape[0]
        # inference: the weights are quantized once, before the steps
        w1 = mx.quantize(upload(lin["W1"]), rowwise=True, packed=True)
        w2 = mx.quantize(upload(lin["W2"]), rowwise=True, packed=True)
        keep.extend([w1, w2])
        bx = quantize_op("X[%dx%d]" % (T, D), lin["X"], ROW, packed=True)
        hq = torch.empty((T, F), dtype=torch.uint8, device=dev)
        hp = torch.empty((F // 128, T), dtype=torch.int32, device=dev)
        y = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
        keep.extend([hq, hp, y])
        dominant = "fc1 gelu mxfp8-out %dx%dx%d" % (T, F, D)
        ops.append(Op("gemm", dominant, lambda st: mx.mxfp8_gemm_mxfp8_out(
            bx["q"], bx["p"], w1["q_row"], w1["p_row"], None, hq, F, hp, T, F, D, mx.MXFP8_GEMM_GELU, stream=st),
            2.0 * T * F * D))
        ops.append(Op("gemm", "fc2 %dx%dx%d" % (T, D, F), lambda st: mx.mxfp8_gemm_ex(
            hq, hp, w2["q_row"], w2["p_row"], y, D, T, D, F, 0, stream=st), 2.0 * T * D * F))
        desc = ("GELU MLP inference forward, tokens %d, d_model %d, d_ff %d: X N(0,1), W1 and W2 N(0,0.02) "
                "quantized once before the steps; per step the rowwise quantize of X into packed scales, FC1 "
                "GEMM with the GELU epilogue writing its output as MXFP8 (rowwise codes + packed scale words), "
                "FC2 GEMM on those codes with BF16 output" % (T, D, F))
    elif workload == "moe_fwd":
        d = workloads.moe()
        w2h = workloads.moe_fc2()["W2"]
        host = dict(d, W2=w2h)
        G, NB, K = d["W"].shape
        N = NB // 2
        D = w2h.shape[1]
        Mt = d["X"].shape[0]
        # inference: the expert weights are quantized once, before the steps
        w1 = mx.quantize(upload(d["W"].reshape(G * NB, K)), rowwise=True, packed=True)
        w2 = mx.quantize(upload(w2h.reshape(G * D, N)), rowwise=True, packed=True)
        keep.extend([w1, w2])
        bx = quantize_op("X[%dx%d]" % (Mt, K), d["X"], ROW, packed=True)
        off = torch.from_numpy(d["offsets"]).to(dev)
        hq = torch.empty((Mt, N), dtype=torch.uint8, device=dev)
        hp = torch.empty((N // 128, Mt), dtype=torch.int32, device=dev)
        y = torch.empty((Mt, D), dtype=torch.bfloat16, device=dev)
        keep.extend([off, hq, hp, y])
        tokens = int(d["offsets"][-1] - d["offsets"][0])
        dominant = "grouped fc1 swiglu mxfp8-out %dx%dx%d G=%d" % (Mt, NB, K, G)
        ops.append(Op("gemm", dominant, lambda st: mx.mxfp8_grouped_gemm_mxfp8_out(
            bx["q"], bx["p"], w1["q_row"], w1["p_row"], off, G, None, hq, N, hp, Mt, N, K, mx.MXFP8_GEMM_SWIGLU,
            stream=st), 2.0 * tokens * NB * K))
        ops.append(Op("gemm", "grouped fc2 %dx%dx%d G=%d" % (Mt, D, N, G), lambda st: mx.mxfp8_grouped_gemm_ex(
            hq, hp, w2["q_row"], w2["p_row"], off, G, y, D, Mt, D, N, 0, stream=st), 2.0 * tokens * D * N))
        desc = ("MoE block inference forward over %d experts (token counts %s): X[%dx%d] N(0,1); W1[%d][%dx%d] "
                "(per expert %d gate rows, then %d up rows) and W2[%d][%dx%d] N(0,0.02) quantized once before the "
                "steps; per step the rowwise quantize of X into packed scales, the grouped first projection with "
                "the SwiGLU epilogue writing MXFP8 [%dx%d], the grouped second projection on those codes with "
                "BF16 output [%dx%d]" % (G, np.diff(d["offsets"]).tolist(), Mt, K, G, NB, K, N, N, G, D, N, Mt, N,
                                         Mt, D))
    elif workload == "moe_swiglu":
        d = workloads.moe()
        host = d
        G, NB, K = d["W"].shape
        N = NB // 2
        Mt = d["X"].shape[0]
        bx = quantize_op("X[%dx%d]" % (Mt, K), d["X"], ROW, packed=True)
        bw = quantize_op("W[%dx%dx%d]" % (G, NB, K), d["W"].reshape(G * NB, K), ROW, packed=True)
        off = torch.from_numpy(d["offsets"]).to(dev)
        c = torch.empty((Mt, N), dtype=torch.bfloat16, device=dev)
        keep.extend([c, off])
        tokens = int(d["offsets"][-1] - d["offsets"][0])
        dominant = "grouped swiglu %dx%dx%d G=%d" % (Mt, NB, K, G)
        ops.append(Op("gemm", dominant, lambda st: mx.mxfp8_grouped_gemm_ex(
            bx["q"], bx["p"], bw["q"], bw["p"], off, G, c, N, Mt, N, K, mx.MXFP8_GEMM_SWIGLU, stream=st),
            2.0 * tokens * NB * K))
        desc = ("MoE first projection with the SwiGLU epilogue: X[%dx%d] and W[%d][%dx%d] (per expert %d gate rows, "
                "then %d up rows) rowwise into packed scales, ragged grouped GEMM over %d experts (token counts %s) "
                "writing SiLU(X W_gate^T) * (X W_up^T) [%dx%d]"
                % (Mt, K, G, NB, K, N, N, G, np.diff(d["offsets"]).tolist(), Mt, N))
    elif workload == "moe_sqrelu":
        d = workloads.moe()
        host = d
        G, N, K = d["W"].shape
        Mt = d["X"].shape[0]
        bx = quantize_op("X[%dx%d]" % (Mt, K), d["X"], ROW, packed=True)
        bw = quantize_op("W[%dx%dx%d]" % (G, N, K), d["W"].reshape(G * N, K), ROW, packed=True)
        off = torch.from_numpy(d["offsets"]).to(dev)
        c = torch.empty((Mt, N), dtype=torch.bfloat16, device=dev)
        keep.extend([c, off])
        tokens = int(d["offsets"][-1] - d["offsets"][0])
        dominant = "grouped relu^2 %dx%dx%d G=%d" % (Mt, N, K, G)
        ops.append(Op("gemm", dominant, lambda st: mx.mxfp8_grouped_gemm_ex(
            bx["q"], bx["p"], bw["q"], bw["p"], off, G, c, N, Mt, N, K, mx.MXFP8_GEMM_SQRELU, stream=st),
            2.0 * tokens * N * K))
        desc = ("MoE first projection with the squared-ReLU epilogue: X[%dx%d] and W[%d][%dx%d] rowwise into "
                "packed scales, ragged grouped GEMM over %d experts (token counts %s) writing relu(XW^T)^2"
                % (Mt, K, G, N, K, G, np.diff(d["offsets"]).tolist()))
    else:  # moe
        d = workloads.moe()
        host = d
        G, N, K = d["W"].shape
        Mt = d["X"].shape[0]
        bx = quantize_op("X[%dx%d]" % (Mt, K), d["X"], ROW)
        bw = quantize_op("W[%dx%dx%d]" % (G, N, K), d["W"].reshape(G * N, K), ROW)
        off = torch.from_numpy(d["offsets"]).to(dev)
        c = torch.empty((Mt, N), dtype=torch.bfloat16, device=dev)
        keep.extend([c, off])
        tokens = int(d["offsets"][-1] - d["offsets"][0])
        dominant = "grouped %dx%dx%d G=%d" % (Mt, N, K, G)
        ops.append(Op("gemm", dominant, lambda st: mx.mxfp8_grouped_gemm(
            bx["q"], bx["p"], bw["q"], bw["p"], off, G, c, N, Mt, N, K, stream=st), 2.0 * tokens * N * K))
        desc = ("grouped MoE: X[%dx%d] and W[%d][%dx%d] rowwise, ragged grouped GEMM over %d experts with "
                "token counts %s" % (Mt, K, G, N, K, G, np.diff(d["offsets"]).tolist()))
    return ops, keep, dominant, desc, host


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mxfp8_block_scaled_quantize_amd as mx

    if not os.path.exists(mx.LIB_PATH):
        from mxfp8_block_scaled_quantize_amd import build as mxbuild
        mxbuild.build()
    mx.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    ops, keep, dominant, desc, host = build_ops(args.workload, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    # In the timed steps each GEMM launch is bracketed by HIP events on its
    # stream, and each run of consecutive quantize / packing launches by one
    # pair (per-launch markers between the short launches would add ~3 % of
    # idle time to the step).  Per-launch times of those short kernels come
    # from a separate pass after the timed region.
    groups = []
    for op in ops:
        if op.kind == "gemm" or not groups or groups[-1][0].kind == "gemm":
            groups.append([op])
        else:
            groups[-1].append(op)

    def step(ev=None, per_launch=False):
        for grp in (groups if not per_launch else [[op] for op in ops]):
            if ev is None:
                for op in grp:
                    op.fn(stream)
                continue
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for op in grp:
                op.fn(stream)
            e1.record(stream)
            ev.append((tuple(grp), e0, e1))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    detail = []
    for _ in range(min(args.steps, 10)):
        step(detail, per_launch=True)
    torch.cuda.synchronize()

    def durations(evs):
        dur = {}
        for grp, e0, e1 in evs:
            dur.setdefault(tuple(id(op) for op in grp), []).append(e0.elapsed_time(e1))
        return dur

    def stats(v):
        return {"ms": float(np.mean(v)), "ms_median": float(np.median(v)), "ms_min": float(np.min(v)),
                "ms_max": float(np.max(v)), "n": len(v)}

    timed_d = durations(events)
    timed = {k: float(np.mean(v)) for k, v in timed_d.items()}
    per = {k[0]: stats(v) for k, v in durations(detail).items()}
    for k, v in timed_d.items():     # GEMMs: the timed-region numbers
        if len(k) == 1:
            per[k[0]] = stats(v)
    avg = {k: v["ms"] for k, v in per.items()}
    short_block = [(k, v) for k, v in timed.items() if len(k) > 1 or
                   [op for op in ops if id(op) == k[0]][0].kind != "gemm"]

    def rounded(st):
        return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in st.items()}

    total_flops = sum(op.work for op in ops if op.kind == "gemm")
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    by_id = {id(op): op for op in ops}
    block_report = []
    for k, t in short_block:
        work = sum(by_id[i].work for i in k)
        block_report.append({"launches": [by_id[i].kind + " " + by_id[i].label for i in k], "ms": round(t, 4),
                             "gbs": round(work / (t * 1e-3) / 1e9, 1)})
    gemm_report, quant_report, pack_report = {}, {}, {}
    for op in ops:
        t = avg[id(op)]
        if op.kind == "gemm":
            tf = op.work / (t * 1e-3) / 1e12
            gemm_report[op.label] = dict(rounded(per[id(op)]), tflops=round(tf, 1),
                                         frac_fp8_peak=round(tf / FP8_PEAK_TFLOPS, 4),
                                         tflops_at_median=round(op.work / (per[id(op)]["ms_median"] * 1e-3) / 1e12, 1))
        else:
            gbs = op.work / (t * 1e-3) / 1e9
            rep = quant_report if op.kind == "quantize" else pack_report
            rep[op.label] = dict(rounded(per[id(op)]), gbs=round(gbs, 1), frac_hbm_peak=round(gbs / HBM_PEAK_GBS, 4),
                                 gbs_at_median=round(op.work / (per[id(op)]["ms_median"] * 1e-3) / 1e9, 1))

    dom = [op for op in ops if op.kind == "gemm" and op.label == dominant][0]
    dom_t = avg[id(dom)]
    achieved = dom.work / (dom_t * 1e-3) / 1e12
    prof = profiled_traffic("gemm:" + dominant.replace(" ", ":"))
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": prof[0] if prof else None,
                "kernel": "mxfp8 gemm " + dominant, "flops_per_launch": dom.work}
    roofline.update(rounded(per[id(dom)]))
    if prof:
        roofline["traffic_unit"] = "bytes per launch (HBM side, calibrated FETCH_SIZE + WRITE_SIZE)"
        roofline["traffic_source"] = "profiles/" + prof[1]

    # the quantizer's roofline: its largest launch of the step (per-launch HIP
    # events), and all quantize / packing launches as timed inside the steps
    qops = [op for op in ops if op.kind == "quantize"]
    qroof = None
    if qops:
        qdom = max(qops, key=lambda op: op.work)
        qt = avg[id(qdom)]
        qgbs = qdom.work / (qt * 1e-3) / 1e9
        qprof = profiled_traffic("quantize:" + qdom.label.replace(" ", ":"), QUANTIZE_SOURCES)
        in_steps = sum(sum(by_id[i].work for i in k) for k, _ in short_block)
        in_steps_ms = sum(t for _, t in short_block)
        qroof = {"bound": "hbm", "achieved": round(qgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(qgbs / HBM_PEAK_GBS, 4), "traffic": qprof[0] if qprof else None,
                 "kernel": "mxfp8 quantize " + qdom.label, "bytes_per_launch": qdom.work,
                 "all_short_launches_in_steps_gbs": round(in_steps / (in_steps_ms * 1e-3) / 1e9, 1)}
        qroof.update(rounded(per[id(qdom)]))
        if qprof:
            qroof["traffic_source"] = "profiles/" + qprof[1]

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": desc, "gemm_flops_per_step": total_flops},
        "roofline": roofline,
        "quantize_roofline": qroof,
        "gemm": gemm_report,
        "quantize": quant_report,
        "pack": pack_report,
        "short_launch_blocks": block_report,
        "launch_order": [op.kind + " " + op.label for op in ops],
        "timing_note": "gemm: HIP events per launch in the timed steps; quantize / pack: per-launch events in a "
                       "separate pass after them (%d steps); ms = mean, with median, min and max; "
                       "short_launch_blocks: the same launches as timed in the steps" % min(args.steps, 10),
    }
    # the register-only MFMA reference first, right after the timed region (as
    # the GEMM ran), then the vendor GEMM
    if not args.no_mfma_calibration:
        result["mfma_calibration"] = mfma_calibration(torch, stream, dominant, dom.work, args.steps, args.warmup,
                                                      achieved)
    if not args.no_vendor_reference:
        result["vendor_reference"] = vendor_reference(torch, stream, dominant, dom.work, args.steps, args.warmup,
                                                      achieved)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.workload, host, total_flops, args.cpu_seconds)

    print(json.dumps(result))


def vendor_reference(torch, stream, label, flops_per_launch, launches, warmup, gemm_tflops):
    """PyTorch's own MXFP8 GEMM on the dominant GEMM's M x N x K (for a grouped
    GEMM: all routed rows as one dense GEMM of the same FLOPs): torch._scaled_mm
    with E4M3 operands and E8M0 scales per 32-element block (hipBLASLt on
    ROCm), BF16 output, random codes and unit scales, timed with HIP events per
    launch on the bench stream.  A reference only: nothing of this library
    runs in it."""
    import re

    import numpy as np

    m = re.search(r"(\d+)x(\d+)x(\d+)", label)
    M, N, K = (int(v) for v in m.groups())
    if "grouped" in label or "swiglu" in label:
        N = int(round(flops_per_launch / (2.0 * M * K)))   # the dense shape of the same FLOPs
    if not hasattr(torch, "float8_e8m0fnu"):
        return {"skipped": "this PyTorch has no float8_e8m0fnu"}
    g = torch.Generator(device="cuda").manual_seed(7)
    try:
        with torch.cuda.stream(stream):
            a = torch.randn((M, K), device="cuda", generator=g).to(torch.float8_e4m3fn)
            b = torch.randn((N, K), device="cuda", generator=g).to(torch.float8_e4m3fn)
            sa = torch.full((M, K // 32), 127, dtype=torch.uint8, device="cuda").view(torch.float8_e8m0fnu)
            sb = torch.full((N, K // 32), 127, dtype=torch.uint8, device="cuda").view(torch.float8_e8m0fnu)

            def launch():
                return torch._scaled_mm(a, b.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)

            # hipBLASLt's algorithm query has been seen to return INVALID_VALUE
            # now and then for a shape it serves otherwise (a status, no
            # fault): the first call is tried up to three times
            failures = []
            while True:
                try:
                    launch()
                    break
                except RuntimeError as e:
                    failures.append(repr(e)[:120])
                    if len(failures) == 3:
                        raise
            for _ in range(warmup):
                launch()
            torch.cuda.synchronize()
            ev = []
            for _ in range(launches):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                launch()
                e1.record(stream)
                ev.append((e0, e1))
            torch.cuda.synchronize()
    except Exception as e:   # not supported by this PyTorch / hipBLASLt build
        return {"skipped": "torch._scaled_mm with MX block scales failed: %s" % repr(e)[:200]}
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    return {"kernel": "torch._scaled_mm, E4M3 x E4M3 with E8M0 scales per 32 (hipBLASLt), BF16 out, no epilogue",
            "shape": "%dx%dx%d" % (M, N, K), "launches": launches, "ms": round(float(np.mean(ms)), 4),
            "ms_median": round(float(np.median(ms)), 4), "tflops": round(float(np.mean(tf)), 1),
            "frac_fp8_peak": round(float(np.mean(tf)) / FP8_PEAK_TFLOPS, 4),
            "this_library_over_vendor": round(gemm_tflops / float(np.mean(tf)), 3),
            "first_call_failures": len(failures)}


def mfma_calibration(torch, stream, label, flops_per_launch, launches, warmup, gemm_tflops):
    """The register-only MFMA kernel of libmxfp8_calib.so (GEMM-shaped
    workgroups: 4 waves, 256 accumulators and 128 operand registers each,
    random E4M3 codes) with the GEMM's grid: one workgroup per 256 x 256 tile
    of the label's M x N x K (for a grouped GEMM, M is all routed rows, i.e.
    the dense grid of the same FLOPs), each running the tile's K / 64 rounds
    of 16 MFMAs per wave.  Timed with HIP events per launch on the bench
    stream."""
    import re
    import ctypes

    import numpy as np

    from mxfp8_block_scaled_quantize_amd.build import CALIB_PATH
    if not os.path.exists(CALIB_PATH):
        return {"skipped": "libmxfp8_calib.so is not built (build() makes it)"}
    L = ctypes.CDLL(CALIB_PATH)
    P = ctypes.c_void_p
    L.mxfp8_calib_mfma_ceiling.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, P]
    L.mxfp8_calib_mfma_ceiling.restype = ctypes.c_int
    words = L.mxfp8_calib_code_words()
    g = torch.Generator().manual_seed(11)
    c = torch.randint(0, 254, (4 * words,), generator=g, dtype=torch.int32)
    c = torch.where(c >= 0x7F, c + 1, c).to(torch.uint8)          # every E4M3 code except the NaNs
    codes = c.view(torch.int32).to("cuda")
    scales = torch.full((128,), 0x77777777, dtype=torch.int32, device="cuda")   # 2^-8: sums stay finite
    m = re.search(r"(\d+)x(\d+)x(\d+)", label)
    if m:
        M, N, K = (int(v) for v in m.groups())
        blocks = ((M + 255) // 256) * ((N + 255) // 256)
        iters = max(1, K // 128)
    else:
        blocks = 1024
        iters = max(1, int(round(flops_per_launch / (blocks * 4 * 32 * 2.0 * 32 * 32 * 64))))
    per_iter = blocks * 4 * 32 * 2.0 * 32 * 32 * 64
    out = torch.empty((blocks * 256,), dtype=torch.float32, device="cuda")

    def launch():
        rc = L.mxfp8_calib_mfma_ceiling(codes.data_ptr(), scales.data_ptr(), out.data_ptr(), blocks, iters,
                                        stream.cuda_stream)
        if rc != 0:
            raise RuntimeError("calibration launch failed (hipError %d)" % rc)

    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    ev = []
    for _ in range(launches):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("calibration sums are not finite")
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    tf = per_iter * iters / (ms * 1e-3) / 1e12
    return {"kernel": "mfma_ceiling_kernel (register-only scaled FP8 MFMA)", "blocks": blocks, "iters": iters,
            "flops_per_launch": per_iter * iters, "launches": launches, "ms": round(float(np.mean(ms)), 4),
            "ms_median": round(float(np.median(ms)), 4), "tflops": round(float(np.mean(tf)), 1),
            "tflops_at_median": round(per_iter * iters / (float(np.median(ms)) * 1e-3) / 1e12, 1),
            "frac_fp8_peak": round(float(np.mean(tf)) / FP8_PEAK_TFLOPS, 4),
            "gemm_over_ceiling": round(gemm_tflops / float(np.mean(tf)), 4)}


def oracle_step(workload, h):
    """One step of the workload run by the CPU oracle on the same inputs: the
    same quantizations (scale packing where the GPU step writes packed words),
    dbias and activations where the GPU fuses them, and every GEMM in fp64 in
    1024-row panels.  Returns the step callable and a description."""
    import numpy as np

    import oracle
    P = 1024

    def both(x):
        q, s = oracle.quantize_rowwise(x)
        qT, sT = oracle.quantize_colwise(x)
        oracle.pack_scales(s)
        oracle.pack_scales(sT)
        return q, s, qT, sT

    def rowp(x):
        q, s = oracle.quantize_rowwise(x)
        oracle.pack_scales(s)
        return q, s

    if workload == "stress":
        def step():
            qa, sa, _, _ = both(h["A"])
            qb, sb = rowp(h["B"])
            oracle.gemm_tn(qa, sa, qb, sb, panel=P)
        return step, ("rowwise + columnwise quantize of A[32768x8192], rowwise B[8192x8192], scale packing, "
                      "fp64 GEMM 32768x8192x8192")
    if workload == "dense":
        def step():
            for a, b in (("X", "W"), ("A", "B")):
                oracle.gemm_tn(*rowp(h[a]), *rowp(h[b]), panel=P)
        return step, ("rowwise quantize of X, W, A, B, scale packing, fp64 GEMMs 8192x14336x4096 and "
                      "8192x8192x8192")
    if workload == "backward":
        def step():
            _, _, qdT, sdT = both(h["dY"])
            oracle.dbias(h["dY"])
            qxT, sxT = oracle.quantize_colwise(h["X"])
            oracle.pack_scales(sxT)
            oracle.gemm_tn(qdT, sdT, qxT, sxT, panel=P)
        return step, ("rowwise + columnwise quantize and dbias of dY[16384x4096], columnwise X, scale packing, "
                      "fp64 wgrad 4096x4096x16384")
    if workload in ("moe", "moe_sqrelu", "moe_swiglu"):
        def step():
            qx, sx = rowp(h["X"])
            ws = [rowp(w) for w in h["W"]]
            c = oracle.grouped_gemm_tn(qx, sx, np.stack([q for q, _ in ws]), np.stack([s for _, s in ws]),
                                       h["offsets"], panel=P)
            if workload == "moe_sqrelu":
                oracle.sqrelu_epilogue(c)
            if workload == "moe_swiglu":
                oracle.swiglu_epilogue(c)
        epi = {"moe": "", "moe_sqrelu": " with the relu^2 epilogue", "moe_swiglu": " with the SwiGLU epilogue"}
        return step, ("rowwise quantize of X[16384x4096] and W[8][14336x4096], scale packing, fp64 grouped "
                      "GEMM" + epi[workload])
    if workload == "linear":
        def step():
            qx, sx, qxT, sxT = both(h["X"])
            qw, sw, qwT, swT = both(h["W"])
            qd, sd, qdT, sdT = both(h["dY"])
            oracle.gemm_tn(qx, sx, qw, sw, panel=P)
            oracle.gemm_tn(qd, sd, qwT, swT, panel=P)
            oracle.gemm_tn(qdT, sdT, qxT, sxT, panel=P)
        return step, "row+col quantize of X, W, dY, scale packing, fp64 fprop, dgrad and wgrad"
    if workload == "moe_fwd":
        G = h["W"].shape[0]
        w1 = [rowp(w) for w in h["W"]]
        w2 = [rowp(w) for w in h["W2"]]
        q1, s1 = np.stack([q for q, _ in w1]), np.stack([s for _, s in w1])
        q2, s2 = np.stack([q for q, _ in w2]), np.stack([s for _, s in w2])

        def step():
            qx, sx = rowp(h["X"])
            hv = oracle.swiglu_epilogue(oracle.grouped_gemm_tn(qx, sx, q1, s1, h["offsets"], panel=P))
            qh, sh = oracle.quantize_rowwise_values(np.nan_to_num(hv).astype(np.float32))
            oracle.pack_scales(sh)
            oracle.grouped_gemm_tn(qh, sh, q2, s2, h["offsets"], panel=P)
        return step, ("rowwise quantize of X with scale packing, fp64 grouped first projection, SwiGLU, rowwise "
                      "quantize of the result with scale packing, fp64 grouped second projection (expert weights "
                      "quantized once, outside the steps)")
    if workload == "mlp_fwd":
        q1, s1 = rowp(h["W1"])
        q2, s2 = rowp(h["W2"])

        def step():
            qx, sx = rowp(h["X"])
            hv = oracle.gelu_epilogue(oracle.gemm_tn(qx, sx, q1, s1, panel=P)).astype(np.float32)
            qh, sh = oracle.quantize_rowwise_values(hv)
            oracle.pack_scales(sh)
            oracle.gemm_tn(qh, sh, q2, s2, panel=P)
        return step, ("rowwise quantize of X with scale packing, fp64 FC1 GEMM, GELU, rowwise quantize of the "
                      "result with scale packing, fp64 FC2 GEMM (weights quantized once, outside the steps)")
    if workload in ("mlp", "mlp_gelu"):
        act, dact = ((oracle.act_gelu, oracle.dact_gelu) if workload == "mlp_gelu"
                     else (oracle.act_sqrelu, oracle.dact_sqrelu))

        def step():
            qx, sx, qxT, sxT = both(h["X"])
            q1, s1, q1T, s1T = both(h["W1"])
            q2, s2, q2T, s2T = both(h["W2"])
            qy, sy, qyT, syT = both(h["dY"])
            oracle.gemm_tn(qx, sx, q1, s1, panel=P)                 # fc1
            a = act(h["H"]).astype(np.float32)
            qa, sa = oracle.quantize_rowwise_values(a)
            qaT, saT = oracle.quantize_colwise_values(a)
            oracle.gemm_tn(qa, sa, q2, s2, panel=P)                 # fc2
            oracle.gemm_tn(qy, sy, q2T, s2T, panel=P)               # fc2 dgrad
            oracle.gemm_tn(qyT, syT, qaT, saT, panel=P)             # fc2 wgrad
            g = dact(h["dA"], h["H"]).astype(np.float32)
            qg, sg = oracle.quantize_rowwise_values(g)
            qgT, sgT = oracle.quantize_colwise_values(g)
            oracle.dbias_values(g)
            oracle.gemm_tn(qg, sg, q1T, s1T, panel=P)               # fc1 dgrad
            oracle.gemm_tn(qgT, sgT, qxT, sxT, panel=P)             # fc1 wgrad
        return step, ("row+col quantize of X, W1, W2, dY, the %s activation and its backward (on the "
                      "full-size stand-ins for the GEMM outputs H and dA) quantized row+col (+dbias), six fp64 "
                      "GEMMs" % ("GELU" if workload == "mlp_gelu" else "relu^2"))
    raise ValueError(workload)


def cpu_baseline(workload, host, flops_per_step, min_seconds):
    """The CPU oracle running whole steps of the same workload on the host
    cores until min_seconds have passed (at least one step).  Reported as GEMM
    TFLOP/s of the step, like ``value``."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    step, what = oracle_step(workload, host)
    steps, times = 0, []
    t0 = time.perf_counter()
    while True:
        ts = time.perf_counter()
        step()
        times.append(time.perf_counter() - ts)
        steps += 1
        t1 = time.perf_counter()
        if t1 - t0 >= min_seconds:
            break
    import numpy as np
    return {"value": round(steps * flops_per_step / (t1 - t0) / 1e12, 5), "unit": "TFLOP/s",
            "cores": int(max(oracle.num_threads(), blas_threads)), "kind": "oracle",
            "omp_threads": int(oracle.num_threads()), "blas_threads": int(blas_threads),
            "host_cpu_count": os.cpu_count(),
            "seconds": round(t1 - t0, 2), "steps": steps, "step_s_median": round(float(np.median(times)), 3),
            "sample": "%d whole step(s) of the same workload on the host: %s" % (steps, what)}


if __name__ == "__main__":
    main()
