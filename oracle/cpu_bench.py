"""Time the CPU oracle on a bounded sample of a workload (the benchmark's CPU-baseline leg).

Runs in its own process (no torch, no GPU):  python -m oracle.cpu_bench --workload prefill
Prints one JSON object.  ``--part`` picks what is timed, on chunks of activation rows added
until about ``--seconds`` of CPU work has been timed:

  layer  the per-call work of the layer: the oracle's MX quantization of the rows, their
         dequantization, and the fp64 product with the (already dequantized) weight; the
         weight's quantization and dequantization are load-time work, done once before the
         clock starts, as the prepack is on the GPU.  Reported in TFLOP/s (2 M N K / time).
  quant  the oracle's MX quantization of the rows alone, in GB/s of the quantizer's
         algorithmic bytes (2 + 1 + 1/32 bytes per element).
  gemm   the fp64 product of dequantized rows with the dequantized weight alone, in GFLOP/s.

The thread count is the oracle's OpenMP default (OMP_NUM_THREADS sets it); ``cores`` reports
the threads used, ``cpu_model`` the host's processor name.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from mx_block_scaled_amd import synth  # noqa: E402


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--part", choices=["layer", "quant", "gemm"], default="layer")
    ap.add_argument("--seconds", type=float, default=12.0)
    ap.add_argument("--chunk", type=int, default=8)
    a = ap.parse_args()
    d = synth.make(a.workload, with_w=a.part != "quant")
    M, N, K = d["M"], d["N"], d["K"]
    wfmt = 2 if a.workload == "mxfp6" else 0
    wd = bias = None
    if a.part != "quant":
        wq, ws = oracle.quantize(d["w"], wfmt)
        wd = oracle.dequantize(wq, ws, wfmt)
        bias = None if d["bias"] is None else oracle.bf16_to_f64(d["bias"])
    chunk = a.chunk if a.part != "quant" else max(a.chunk, 64)
    # rows are taken in chunks from the top; the quantizer alone is fast enough to pass over
    # all M rows within the budget, so it wraps around to the first row again
    done_rows, cur = 0, 0
    t_total = 0.0
    while t_total < a.seconds and (a.part == "quant" or cur < M):
        r1 = min(M, cur + chunk)
        xs = np.ascontiguousarray(d["x"][cur:r1])
        if a.part == "gemm":
            q, s = oracle.quantize(xs, oracle.E4M3)
            xd = oracle.dequantize(q, s, oracle.E4M3)
            t0 = time.perf_counter()
            oracle.matmul_nt(xd, wd, bias)
        else:
            t0 = time.perf_counter()
            q, s = oracle.quantize(xs, oracle.E4M3)
            if a.part == "layer":
                xd = oracle.dequantize(q, s, oracle.E4M3)
                oracle.matmul_nt(xd, wd, bias)
        t_total += time.perf_counter() - t0
        done_rows += r1 - cur
        cur = r1 % M if a.part == "quant" else r1
    if a.part == "quant":
        val, unit = 3.03125 * done_rows * K / t_total / 1e9, "GB/s"
    elif a.part == "gemm":
        val, unit = 2.0 * done_rows * N * K / t_total / 1e9, "GFLOP/s"
    else:
        val, unit = 2.0 * done_rows * N * K / t_total / 1e12, "TFLOP/s"
    what = {"layer": "quantize + dequantize + fp64 product with the pre-dequantized weight",
            "quant": "MX quantization (E8M0 scale + E4M3 codes)",
            "gemm": "fp64 product of dequantized rows with the pre-dequantized weight"}[a.part]
    print(json.dumps({
        "value": val, "unit": unit, "cores": oracle.threads(), "kind": "oracle",
        "seconds": t_total, "cpu_model": cpu_model(), "part": a.part,
        "sample": "%d activation rows of the %s workload (%dx%dx%d): %s"
                  % (done_rows, a.workload, M, N, K, what),
    }))


if __name__ == "__main__":
    main()
