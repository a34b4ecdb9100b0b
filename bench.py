"""Benchmark of the MXFP8 hot path on one MI355X.

One step is the dense linear-layer workload: X BF16[8192x4096] ~ N(0,1) and
W BF16[14336x4096] ~ N(0,0.02), plus the square A, B BF16[8192x8192]:
rowwise MXFP8 quantize of all four, scale packing, then the TN GEMMs
8192x14336x4096 and 8192x8192x8192 with BF16 output.  Inputs are resident in
HBM before timing starts.

Printed: one JSON line.  ``value`` is the end-to-end GEMM throughput of the
step (GEMM FLOPs / wall time of the whole step, quantize and packing
included).  ``roofline`` is the dominant kernel (the GEMM at 8192x14336x4096)
against the FP8 MFMA peak, timed with HIP events on its stream;
``quantize`` reports the rowwise quantizer against HBM peak;
``cpu_baseline`` is the CPU oracle on a bounded sample of the same work.
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
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU-oracle time: whole oracle steps are repeated until reached")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one plain 256 MiB device copy (reference for HBM byte counters)")
    return p.parse_args()


def gemm_source_hash():
    """Hash of the sources that define the GEMM kernel (profile traffic is tied to it)."""
    import hashlib
    h = hashlib.sha256()
    for f in ("mxfp8_block_scaled_quantize_amd/csrc/gemm.hip", "mxfp8_block_scaled_quantize_amd/csrc/mx_device.h"):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel_key):
    """HBM-side bytes per launch from the rocprofv3 summaries in profiles/, or None
    when no summary was taken for the current GEMM sources."""
    src = gemm_source_hash()
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    for name in sorted(os.listdir(pdir)):
        with open(os.path.join(pdir, name)) as fh:
            for line in fh:
                parts = line.split()
                if len(parts) >= 5 and parts[0] == "traffic" and " ".join(parts[1:3]) == kernel_key \
                        and parts[3] == "src=" + src:
                    kv = dict(p.split("=", 1) for p in parts[4:] if "=" in p)
                    return int(kv["read_bytes"]) + int(kv["write_bytes"]), name
    return None


def quant_bytes(rows, cols):
    """Algorithmic bytes of a rowwise quantize: read 2 B, write 1 + 1/32 B per element."""
    return rows * cols * (2 + 1 + 1.0 / 32)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mxfp8_block_scaled_quantize_amd as mx
    import workloads

    if not os.path.exists(mx.LIB_PATH):
        from mxfp8_block_scaled_quantize_amd import build as mxbuild
        mxbuild.build()
    mx.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    lin = workloads.dense_linear()
    sq = workloads.dense_square()
    host = {"X": lin["X"], "W": lin["W"], "A": sq["A"], "B": sq["B"]}
    bufs = {}
    for name, bits in host.items():
        R, C = bits.shape
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        bufs[name] = {
            "x": x, "R": R, "C": C,
            "q": torch.empty((R, C), dtype=torch.uint8, device=dev),
            "s": torch.empty((R, C // 32), dtype=torch.uint8, device=dev),
            "p": torch.empty((C // 128, R), dtype=torch.int32, device=dev),
        }
    gemms = [("X", "W"), ("A", "B")]
    outs = [torch.empty((bufs[a]["R"], bufs[b]["R"]), dtype=torch.bfloat16, device=dev) for a, b in gemms]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(ev=None):
        for name, b in bufs.items():
            if ev is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            mx.mxfp8_quantize(b["x"], b["R"], b["C"], b["C"], mx.MXFP8_ROWWISE, b["q"], b["s"], stream=stream)
            if ev is not None:
                e1 = torch.cuda.Event(enable_timing=True)
                e1.record(stream)
            mx.mxfp8_pack_scales(b["s"], b["R"], b["C"], b["C"] // 32, b["p"], stream=stream)
            if ev is not None:
                e2 = torch.cuda.Event(enable_timing=True)
                e2.record(stream)
                ev.append(("quantize", name, e0, e1))
                ev.append(("pack", name, e1, e2))
        for (an, bn), c in zip(gemms, outs):
            a, b = bufs[an], bufs[bn]
            if ev is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            mx.mxfp8_gemm(a["q"], a["p"], b["q"], b["p"], c, b["R"], a["R"], b["R"], a["C"], stream=stream)
            if ev is not None:
                e1 = torch.cuda.Event(enable_timing=True)
                e1.record(stream)
                ev.append(("gemm", an + bn, e0, e1))

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

    dur = {}
    for kind, name, e0, e1 in events:
        dur.setdefault((kind, name), []).append(e0.elapsed_time(e1))
    avg = {k: float(np.mean(v)) for k, v in dur.items()}

    gemm_flops = {an + bn: 2.0 * bufs[an]["R"] * bufs[bn]["R"] * bufs[an]["C"] for an, bn in gemms}
    total_flops = sum(gemm_flops.values())
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    gemm_report = {}
    for key, fl in gemm_flops.items():
        t = avg[("gemm", key)]
        tf = fl / (t * 1e-3) / 1e12
        M, N, K = bufs[key[0]]["R"], bufs[key[1]]["R"], bufs[key[0]]["C"]
        gemm_report["%dx%dx%d" % (M, N, K)] = {"ms": round(t, 4), "tflops": round(tf, 1),
                                              "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)}
    quant_report = {}
    for name, b in bufs.items():
        t = avg[("quantize", name)]
        gbs = quant_bytes(b["R"], b["C"]) / (t * 1e-3) / 1e9
        quant_report["%s[%dx%d]" % (name, b["R"], b["C"])] = {
            "ms": round(t, 4), "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "pack_ms": round(avg[("pack", name)], 4)}

    dom_t = avg[("gemm", "XW")]
    dom_flops = gemm_flops["XW"]
    achieved = dom_flops / (dom_t * 1e-3) / 1e12
    prof = profiled_traffic("gemm 8192x14336x4096")
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": prof[0] if prof else None,
                "kernel": "mxfp8 gemm 8192x14336x4096", "ms": round(dom_t, 4)}
    if prof:
        roofline["traffic_unit"] = "bytes per launch (HBM side, calibrated FETCH_SIZE + WRITE_SIZE)"
        roofline["traffic_source"] = "profiles/" + prof[1]

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
        "config": {"workload": "dense linear layer: rowwise MXFP8 quantize of X[8192x4096], W[14336x4096], "
                               "A[8192x8192], B[8192x8192] + scale packing + TN GEMMs 8192x14336x4096 and "
                               "8192x8192x8192, BF16 out",
                   "global_batch": 8192, "gemm_flops_per_step": total_flops},
        "roofline": roofline,
        "gemm": gemm_report,
        "quantize": quant_report,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(host, args.cpu_seconds)

    print(json.dumps(result))


def cpu_baseline(host, min_seconds):
    """The CPU oracle on the same step: rowwise quantize of X, W, A, B, scale
    packing, and the two GEMMs in fp64; whole steps are repeated until
    min_seconds have passed.  Reported as GEMM TFLOP/s, like ``value``."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    flops = 2.0 * (8192 * 14336 * 4096 + 8192 * 8192 * 8192)
    steps = 0
    t0 = time.perf_counter()
    while True:
        q = {name: oracle.quantize_rowwise(bits) for name, bits in host.items()}
        _ = [oracle.pack_scales(s) for _, s in q.values()]
        for a, b in (("X", "W"), ("A", "B")):
            c = oracle.gemm_tn(*q[a], *q[b])
            del c
        steps += 1
        t1 = time.perf_counter()
        if t1 - t0 >= min_seconds:
            break
    return {"value": round(steps * flops / (t1 - t0) / 1e12, 5), "unit": "TFLOP/s",
            "cores": int(max(oracle.num_threads(), blas_threads)), "kind": "oracle",
            "seconds": round(t1 - t0, 2), "steps": steps,
            "sample": "%d whole step(s) of the same workload on the host: oracle rowwise quantize of X, W, A, B, "
                      "scale packing, fp64 GEMMs 8192x14336x4096 and 8192x8192x8192" % steps}


if __name__ == "__main__":
    main()
