"""Time the CPU oracle on a bounded sample of a workload (the benchmark's CPU-baseline leg).

Runs in its own process (no torch, no GPU):  python -m oracle.cpu_bench --workload prefill
Prints one JSON object.  What is timed, per sample of activation rows: the oracle's MX
quantization of those rows, their dequantization, and the fp64 product with the (already
dequantized) weight — i.e. the per-call work of the layer; the weight's quantization and
dequantization are load-time work, done once before the clock starts, as the prepack is on the
GPU.  Rows are added in chunks until about ``--seconds`` of CPU work has been timed.
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--seconds", type=float, default=12.0)
    ap.add_argument("--chunk", type=int, default=8)
    a = ap.parse_args()
    d = synth.make(a.workload)
    M, N, K = d["M"], d["N"], d["K"]
    wfmt = 2 if a.workload == "mxfp6" else 0
    wq, ws = oracle.quantize(d["w"], wfmt)
    wd = oracle.dequantize(wq, ws, wfmt)
    bias = None if d["bias"] is None else oracle.bf16_to_f64(d["bias"])
    rows = 0
    t_total = 0.0
    while t_total < a.seconds and rows < M:
        r1 = min(M, rows + a.chunk)
        xs = np.ascontiguousarray(d["x"][rows:r1])
        t0 = time.perf_counter()
        q, s = oracle.quantize(xs, oracle.E4M3)
        xd = oracle.dequantize(q, s, oracle.E4M3)
        oracle.matmul_nt(xd, wd, bias)
        t_total += time.perf_counter() - t0
        rows = r1
    flop = 2.0 * rows * N * K
    print(json.dumps({
        "value": flop / t_total / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
        "kind": "oracle", "seconds": t_total,
        "sample": "%d of %d activation rows of the %s workload (%dx%dx%d): quantize + dequantize"
                  " + fp64 product with the pre-dequantized weight" % (rows, M, a.workload, M, N, K),
    }))


if __name__ == "__main__":
    main()
