#!/usr/bin/env python3
"""bench.py — throughput of the MXFP8 linear layer (activation quantization + block-scaled GEMM)
on one MI355X.

A step is one call of the layer on the prefill workload: x bf16 [4096, 4096] ~ N(0,1), weight
[14336, 4096] (MLP up-projection shape) quantized to E4M3 + E8M0 from N(0, 0.02), no bias, bf16
out, through mxfp8_linear (quantizer kernel + GEMM kernel).  value = 2*M*N*K / step time, in
TFLOP/s, with activation quantization inside the timed step.  Inputs are resident in HBM before
the clock starts; R copies of the inputs/weights/outputs are rotated so the working set exceeds
the 256 MiB Infinity Cache.

Order of a run: the chip is first brought to its steady clock (steps for --settle-ms of GPU
time); the GEMM and quantizer are timed alone (roofline); then W warmup steps and exactly K
timed steps (wall clock between two synchronizations, HIP events alongside), which give
`value`; then the step protocol: 5 loops of >= 100 steps timed with HIP events (median, min).

Also measured and printed in the same JSON line:
  roofline      the GEMM kernel alone (pre-quantized entry), 5 loops of >= 100 launches timed
                with HIP events on the stream it runs on (median): achieved TFLOP/s against
                the 5.0 PFLOP/s dense FP8 peak, and against the attainable peak that the MFMA
                loop of libmxpeaks measures on the same chip; traffic from the committed
                rocprofv3 counter summary while the kernel source still matches it, else null;
  clock         the shader clock the chip runs at under back-to-back GEMMs: a one-wave probe on
                a second stream counts shader-clock cycles against the 100 MHz counter while
                the calls run;
  attainable    the MFMA-loop peaks (FP8 x FP8, FP8 x FP6, FP6 x FP6) and the HBM stream-read
                rate of 1 GiB, measured in this run;
  decode        the decode workload (x [M, 4096], M in {1, 8, 32}, weight [4096, 4096], bias),
                one fused call each, replayed from a HIP graph over 32 rotated weight copies:
                time per call, algorithmic bytes / time against 8 TB/s and against a plain
                read of the same weight bytes replayed the same way (the stream floor); the
                same for M = 64 and 128 (prefill chunks), and every M in batch-invariant mode;
                and M = 1, 8, 32 eight layers per call through the batched entry (time per
                layer);
  other_workloads  outlier activations on the pre-quantized entry (2048 x 6144 x 4096, GEMM
                only), MXFP6 weights (E2M3 and E3M2, 512 x 8192 x 8192, activation quantization
                included) with MXFP8 activations and with MXFP6 activations of the same format
                (both MFMA operands FP6), each over enough rotated sets to exceed the Infinity
                Cache; the fused RMS norm + MXFP8 quantizer on the prefill activations against a
                torch RMS norm followed by the standalone quantizer; the latency of one tiny
                call (16 x 256 x 512) from a HIP graph; the batched layer.  Each is timed after
                --settle-ms / 2 of its own calls, as the median of 5 loops (HIP events);
  cpu_baseline  the CPU oracle on bounded samples of the prefill workload (host cores), run in
                separate processes (oracle/cpu_bench.py): the whole layer (value), and the
                quantizer (GB/s) and fp64 GEMM (GFLOP/s) apart, on all cores and on one thread.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --only peaks            (MFMA-loop peaks, stream reads 16 MiB .. 1 GiB)
       python bench.py --only gemm --steps K   (the GEMM alone, for rocprofv3 --pmc passes)
       python bench.py --only decode --steps K (the decode calls, for rocprofv3 --pmc passes)
       python bench.py --only copy             (1 GiB device copy x 3: counter calibration)
"""
import argparse
import ctypes
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA
PEAK_FP6_TFLOPS = 10100.0    # MI355X dense FP6 / FP4 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
MALL_BYTES = 256 << 20


def _gemm_source_hash():
    h = hashlib.sha256()
    for f in ("mx_gemm.hip", "mx_device.h"):
        h.update(open(os.path.join(ROOT, "mx_block_scaled_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def _traffic(kernel_key, n_launch_units=1):
    """HBM bytes per launch from profiles/traffic.json, if the kernel source is unchanged."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        t = json.load(open(p))[kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_sha") != _gemm_source_hash():
        return None
    return t.get("bytes_per_launch")


def _peaks_lib():
    path = os.path.join(ROOT, "mx_block_scaled_amd", "libmxpeaks.so")
    if not os.path.exists(path):
        raise RuntimeError("libmxpeaks.so is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.mxpk_mfma_loop.restype, L.mxpk_mfma_loop.argtypes = I, [I, I, I, I, P, P, P]
    L.mxpk_mfma_chains.restype, L.mxpk_mfma_chains.argtypes = I, []
    L.mxpk_stream_read.restype, L.mxpk_stream_read.argtypes = I, [P, I64, I, I, P, P]
    L.mxpk_clock_probe.restype, L.mxpk_clock_probe.argtypes = I, [I64, P, P]
    L.mxpk_lds_read.restype, L.mxpk_lds_read.argtypes = I, [I, I, I, I, P, P, P]
    L.mxpk_l1_copy.restype, L.mxpk_l1_copy.argtypes = I, [I, P, I, I, I, P, P, P]
    return L


def cu_rates(L):
    """Per-CU data rates of one workgroup per CU (256 workgroups), in bytes per shader clock of
    block 0's loop: LDS reads (16- and 8-byte lanes, 4 / 8 / 16 waves) and global -> CU copies
    from an L2-resident 256 KiB window (16-byte direct-to-LDS, 16-byte into registers, 4-byte
    direct-to-LDS; 16 waves)."""
    import torch
    st = torch.cuda.current_stream().cuda_stream
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    res = {"lds_read_B_per_clk": {}, "l1_copy_B_per_clk": {}}
    iters = 2000
    for width in (16, 8):
        for threads in (256, 512, 1024):
            for _ in range(2):
                assert L.mxpk_lds_read(width, threads, 256, iters, out.data_ptr(), clk.data_ptr(), st) == 0
            torch.cuda.synchronize()
            cyc = clk.cpu().tolist()[0]
            key = "b%d_%dwaves" % (width * 8, threads // 64)
            res["lds_read_B_per_clk"][key] = round(threads * iters * 8 * width / cyc, 1) if cyc else None
    src = torch.full((512 << 10,), 1, dtype=torch.uint8, device="cuda")
    for mode, name, width in ((0, "lds_dma_16B", 16), (1, "vgpr_16B", 16), (2, "lds_dma_4B", 4)):
        for _ in range(2):
            assert L.mxpk_l1_copy(mode, src.data_ptr(), 1024, 256, iters, out.data_ptr(), clk.data_ptr(), st) == 0
        torch.cuda.synchronize()
        cyc = clk.cpu().tolist()[0]
        res["l1_copy_B_per_clk"][name + "_16waves"] = round(1024 * iters * 8 * width / cyc, 1) if cyc else None
    del src
    return res


def clock_under(L, fn, calls, probe_ms):
    """Shader clock (MHz) while fn(i) runs ``calls`` times back to back: a one-wave probe on a
    second stream, launched just before the calls so that it is resident while they run,
    counts the shader-clock cycles (s_memtime) against the 100 MHz counter (s_memrealtime) for
    ``probe_ms``.  (Enqueued behind queued calls instead, the probe started only after the
    quantizer + GEMM steps had drained and read the idle clock.)"""
    import torch
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    assert L.mxpk_clock_probe(int(probe_ms * 1e5), out.data_ptr(), side.cuda_stream) == 0
    for i in range(calls):
        fn(i)
    torch.cuda.synchronize()
    cyc, ticks = out.cpu().tolist()
    return round(cyc / (ticks / 100.0), 1) if ticks > 0 else None


def event_loops(fn, loops=5, iters=100, warm=10):
    """Times ``iters`` back-to-back calls of fn(i) with HIP events on the current stream,
    ``loops`` times: (median, min) microseconds per call."""
    import torch
    stream = torch.cuda.current_stream()
    for i in range(warm):
        fn(i)
    per = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(loops):
        e0.record(stream)
        for i in range(iters):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / iters)
    return statistics.median(per), min(per)


def mfma_peak(L, afmt, bfmt, blocks, iters=20000):
    """(TFLOP/s, shader clock in MHz) of the MFMA loop: blocks x 4 waves x iters x chains
    scaled 16x16x128 MFMAs; the clock from block 0's s_memtime / s_memrealtime stamps."""
    import torch
    out = torch.zeros(4, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    flop = blocks * 4.0 * iters * L.mxpk_mfma_chains() * 2 * 16 * 16 * 128

    def run(_):
        assert L.mxpk_mfma_loop(afmt, bfmt, blocks, iters, out.data_ptr(), clk.data_ptr(), st) == 0

    med, _ = event_loops(run, loops=3, iters=1, warm=1)
    c = clk.cpu().tolist()
    mhz = c[0] / (c[1] / 100.0) if c[1] > 0 else None
    return flop / (med * 1e-6) / 1e12, mhz


def stream_read_us(L, nbytes, sets=None, reps=20, configs=None):
    """Best microseconds per plain read of nbytes over the (unroll, blocks) configs, replayed
    from a HIP graph over enough distinct buffers (>= 2 x the Infinity Cache in all) that the
    reads come from HBM: the same method the decode calls are timed with."""
    import torch
    nbytes = (nbytes + 15) // 16 * 16
    n16 = nbytes // 16
    n = sets or max(1, -(-2 * MALL_BYTES // nbytes))
    if configs is None:
        configs = [(u, max(1, min(16384, -(-n16 // (256 * u * k))))) for u in (4, 8, 16)
                   for k in (1, 2, 4)]
    bufs = [torch.full((nbytes,), j + 1, dtype=torch.uint8, device="cuda") for j in range(n)]
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    per_graph = max(n, 8)
    best = None
    for unroll, blocks in configs:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for j in range(per_graph):
                assert L.mxpk_stream_read(bufs[j % n].data_ptr(), nbytes, blocks, unroll,
                                          out.data_ptr(), s.cuda_stream) == 0
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for j in range(per_graph):
                L.mxpk_stream_read(bufs[j % n].data_ptr(), nbytes, blocks, unroll,
                                   out.data_ptr(), s.cuda_stream)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / (reps * per_graph)
        del g
        if best is None or us < best[0]:
            best = (us, unroll, blocks)
    del bufs
    torch.cuda.empty_cache()
    return best


def measure_peaks(full=False):
    """Attainable peaks of the running chip: MFMA loops (4 and 8 waves per SIMD, the better
    one), plain HBM reads (the best launch shape) and the per-CU LDS and L1 rates."""
    L = _peaks_lib()
    res = {"mfma_TFLOPs": {}, "mfma_clock_MHz": {}}
    for name, af, bf in (("fp8xfp8", 0, 0), ("fp8xfp6", 0, 2), ("fp6xfp6", 2, 2),
                         ("fp8xfp8_32x32x64", 100, 100), ("fp8xfp8_random", 200, 200)):
        # the random-operand loop runs ~30 ms per launch: the chip's power limit takes a few
        # milliseconds to pull the clock down to where it holds
        its = 200000 if af == 200 else 20000
        best = max((mfma_peak(L, af, bf, blocks, iters=its) for blocks in (1024, 2048)),
                   key=lambda r: r[0])
        res["mfma_TFLOPs"][name] = round(best[0], 1)
        res["mfma_clock_MHz"][name] = round(best[1], 1) if best[1] else None
    sizes = [16 << 20, 64 << 20, 256 << 20, 1 << 30] if full else [1 << 30]
    res["stream_read"] = {}
    for b in sizes:
        us, unroll, blocks = stream_read_us(L, b)
        res["stream_read"]["%dMiB" % (b >> 20)] = {"us": round(us, 2),
                                                    "GB/s": round(b / us / 1e3, 1),
                                                    "unroll": unroll, "blocks": blocks}
    res["hbm_GBs"] = res["stream_read"]["1024MiB"]["GB/s"]
    res["per_CU"] = cu_rates(L)
    return res, L


def gemm_only(args, dev):
    """--only gemm for the outlier and MXFP6 workloads: the GEMM alone (pre-quantized entry)
    --steps times over enough rotated operand / output sets to exceed the Infinity Cache, for
    rocprofv3 counter passes."""
    import numpy as np
    import torch
    from mx_block_scaled_amd import mxfp8, synth

    def bf16_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    name = {"outlier": "outlier"}.get(args.workload, "mxfp6")
    d = synth.make(name)
    M, N, K = d["M"], d["N"], d["K"]
    wfmt = "e4m3" if args.workload == "outlier" else args.workload.split("_")[1]
    afmt = wfmt if args.workload.startswith("w6a6") else "e4m3"
    xq, xs = mxfp8.quantize_act_fmt(bf16_dev(d["x"]), afmt)
    wq, ws = mxfp8.quantize_weight(bf16_dev(d["w"]), wfmt)
    pk = mxfp8.prepack_weight(wq, ws, wfmt)
    del wq, ws
    set_bytes = xq.numel() + xs.numel() + pk.numel() + M * N * 2
    R = max(2, -(-2 * MALL_BYTES // set_bytes))
    sets = [(xq.clone(), xs.clone(), pk.clone(), torch.empty((M, N), dtype=torch.bfloat16, device=dev))
            for _ in range(R)]
    for i in range(args.steps):
        a, b, p, y = sets[i % R]
        mxfp8.linear_prequant_fmt(a, b, p, N, K, wfmt, afmt, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"gemm_launches": args.steps, "workload": args.workload, "rotated_sets": R,
                      "M": M, "N": N, "K": K}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the outlier, MXFP6 and tiny workloads")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="CPU time of the whole-layer oracle sample (the split parts take "
                         "a quarter of it each)")
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="GPU time of untimed steps run first, so the chip reaches its steady "
                         "clock before anything is timed")
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "outlier", "mxfp6_e2m3", "mxfp6_e3m2", "w6a6_e2m3",
                             "w6a6_e3m2"],
                    help="with --only gemm: whose GEMM is launched (pre-quantized entry)")
    ap.add_argument("--only", choices=["all", "gemm", "copy", "decode", "peaks"], default="all",
                    help="counter runs: 'gemm' launches only the prefill GEMM (pre-quantized "
                         "entry) --steps times; 'decode' runs the decode calls (M = 1, 8, 32) "
                         "--steps times each over the rotated weights, without a graph; 'copy' "
                         "copies a 1 GiB device buffer 3 times, the calibration of the HBM byte "
                         "counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from mx_block_scaled_amd import mxfp8, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.only == "peaks":
        res, _ = measure_peaks(full=True)
        print(json.dumps(res))
        return

    if args.only == "copy":
        src = torch.full((1 << 30,), 3, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copied_bytes_per_launch": 1 << 30, "launches": 3}))
        return

    if args.only == "decode":
        dd = synth.make("decode32")
        Nd = Kd = 4096
        w0 = torch.from_numpy(dd["w"].view(np.int16)).view(torch.bfloat16).to(dev)
        wq, ws = mxfp8.quantize_weight(w0, "e4m3")
        pk = mxfp8.prepack_weight(wq, ws, "e4m3")
        bias = torch.from_numpy(dd["bias"].view(np.int16)).view(torch.bfloat16).to(dev)
        pks = [pk] + [pk.clone() for _ in range(31)]
        for Md in (1, 8, 32):
            xd = torch.from_numpy(dd["x"][:Md].view(np.int16)).view(torch.bfloat16).to(dev)
            yd = torch.empty((Md, Nd), dtype=torch.bfloat16, device=dev)
            wsd = mxfp8.new_workspace(mxfp8.workspace_bytes(Md, Nd, Kd), dev)
            for i in range(args.steps):
                mxfp8.linear(xd, pks[i % 32], Nd, "e4m3", bias, out=yd, workspace=wsd)
            torch.cuda.synchronize()
        print(json.dumps({"decode_calls_per_M": args.steps, "M": [1, 8, 32], "N": Nd, "K": Kd}))
        return

    if args.only == "gemm" and args.workload != "prefill":
        gemm_only(args, dev)
        return

    # ------------------------------------------------------------ prefill workload
    M, N, K = 4096, 14336, 4096
    d = synth.make("prefill")
    # SHA-256 of the generated bf16 inputs (bit patterns), so a run names its exact data
    inputs_sha = {k: hashlib.sha256(np.ascontiguousarray(d[k]).tobytes()).hexdigest()[:16]
                  for k in ("x", "w")}
    x0 = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    w0 = torch.from_numpy(d["w"].view(np.int16)).view(torch.bfloat16).to(dev)
    wq, ws = mxfp8.quantize_weight(w0, "e4m3")
    packed0 = mxfp8.prepack_weight(wq, ws, "e4m3")
    del w0, wq, ws
    set_bytes = x0.numel() * 2 + packed0.numel() + M * N * 2
    R = max(2, -(-2 * MALL_BYTES // set_bytes))
    if args.only == "gemm":
        # the launches whose HBM counters give roofline.traffic: the same rotation over R
        # operand / output sets as the timed GEMM-alone loop below
        xq, xsc = mxfp8.quantize_act(x0)
        xqs = [xq] + [xq.clone() for _ in range(R - 1)]
        xss = [xsc] + [xsc.clone() for _ in range(R - 1)]
        pks = [packed0] + [packed0.clone() for _ in range(R - 1)]
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
        for i in range(args.steps):
            j = i % R
            mxfp8.linear_prequant(xqs[j], xss[j], pks[j], N, "e4m3", out=ys[j])
        torch.cuda.synchronize()
        print(json.dumps({"gemm_launches": args.steps, "rotated_sets": R, "M": M, "N": N, "K": K}))
        return
    xs_ = [x0] + [x0.clone() for _ in range(R - 1)]
    ps_ = [packed0] + [packed0.clone() for _ in range(R - 1)]
    ys_ = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    wsb = torch.zeros(mxfp8.workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    flop = 2.0 * M * N * K

    def step(i):
        j = i % R
        mxfp8.linear(xs_[j], ps_[j], N, "e4m3", out=ys_[j], workspace=wsb)

    # bring the chip to its steady clock: untimed steps for --settle-ms of GPU time
    t_settle = time.perf_counter()
    n_settle = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for i in range(20):
            step(n_settle + i)
        n_settle += 20
        torch.cuda.synchronize()

    # ------------------------------------------------------------ GEMM kernel alone (roofline)
    xq_, xsc_ = [], []
    for j in range(R):
        q, sc = mxfp8.quantize_act(xs_[j])
        xq_.append(q)
        xsc_.append(sc)
    gemm_us, gemm_us_min = event_loops(
        lambda i: mxfp8.linear_prequant(xq_[i % R], xsc_[i % R], ps_[i % R], N, "e4m3",
                                        out=ys_[i % R]))
    achieved = flop / (gemm_us * 1e-6) / 1e12
    quant_us, quant_us_min = event_loops(lambda i: mxfp8.quantize_act(xs_[i % R]))
    del xq_, xsc_
    quant_bytes = M * K * 2 + M * K + M * K // 32

    # ------------------------------------------------------------ the timed steps (value)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    ms_per_step_events = e0.elapsed_time(e1) / args.steps
    value = flop / (ms_per_step * 1e-3) / 1e12

    # step protocol: 5 loops of >= 100 steps, HIP events
    step_us, step_us_min = event_loops(step, loops=5, iters=max(100, args.steps))

    # ------------------------------------------------------------ attainable peaks
    attainable = None
    try:
        attainable, peaks_lib = measure_peaks(full=False)
    except Exception as e:          # report, never fail the bench line for it
        attainable, peaks_lib = {"error": str(e)[:200]}, None
    att_fp8 = (attainable.get("mfma_TFLOPs") or {}).get("fp8xfp8")
    att_fp8_rand = (attainable.get("mfma_TFLOPs") or {}).get("fp8xfp8_random")
    att_hbm = attainable.get("hbm_GBs")
    # achieved shader clock under the GEMM (a one-wave probe on a second stream, in a separate
    # stretch of calls after the timed loops)
    clock = None
    if peaks_lib is not None:
        xq1, xs1 = mxfp8.quantize_act(xs_[0])
        clock = {
            "gemm_MHz": clock_under(peaks_lib, lambda i: mxfp8.linear_prequant(
                xq1, xs1, ps_[i % R], N, "e4m3", out=ys_[i % R]), 500, 60),
            "mfma_loop_MHz": (attainable.get("mfma_clock_MHz") or {}).get("fp8xfp8"),
            "mfma_loop_random_operands_MHz": (attainable.get("mfma_clock_MHz") or {}).get("fp8xfp8_random"),
            "source": "s_memtime / s_memrealtime of a one-wave probe on a second stream, "
                      "60 ms inside 500 back-to-back calls"}
        del xq1, xs1

    roofline = {
        "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS,
        "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
        "traffic": _traffic("gemm_prefill"),
        "kernel": "k_gemm_pp<0, 0, 7, 4> (pre-quantized entry), %dx%dx%d" % (M, N, K),
        "kernel_us": round(gemm_us, 2), "kernel_us_min": round(gemm_us_min, 2),
        "timing": "HIP events on the launch stream, median of 5 loops of 100 launches",
        "algorithmic_flop_per_launch": flop,
        "attainable_peak": att_fp8,
        "frac_attainable": round(achieved / att_fp8, 4) if att_fp8 else None,
        # the MFMA loop on pseudo-random operands that change every MFMA: the power draw of
        # layer data holds the chip at a lower clock than the constant-operand loop above
        "attainable_peak_random_operands": att_fp8_rand,
        "frac_attainable_random_operands": round(achieved / att_fp8_rand, 4) if att_fp8_rand else None,
    }
    quant_gbs = quant_bytes / (quant_us * 1e-6) / 1e9
    quantizer = {"us": round(quant_us, 2), "us_min": round(quant_us_min, 2),
                 "GB/s": round(quant_gbs, 1), "hbm_frac": round(quant_gbs / PEAK_HBM_GBS, 4),
                 "hbm_frac_attainable": round(quant_gbs / att_hbm, 4) if att_hbm else None}
    step_protocol = {
        "us_median": round(step_us, 2), "us_min": round(step_us_min, 2),
        "TFLOP/s_median": round(flop / step_us / 1e6, 1),
        "TFLOP/s_best": round(flop / step_us_min / 1e6, 1),
        "loops": 5, "steps_per_loop": max(100, args.steps),
        "gemm_plus_quantizer_us": round(gemm_us + quant_us, 2),
        "TFLOP/s_from_gemm_plus_quantizer": round(flop / (gemm_us + quant_us) / 1e6, 1),
        "timed_steps_us_events": round(ms_per_step_events * 1e3, 2),
        "settle_steps": n_settle}

    # ------------------------------------------------------------ decode (HBM-bound)
    decode = None
    if not args.no_decode:
        del xs_, ps_, ys_, wsb
        torch.cuda.empty_cache()
        decode = {}
        dd = synth.make("decode32", M=128)     # rows 0..31: decode; up to 128: chunk sizes
        Nd = Kd = 4096
        w0 = torch.from_numpy(dd["w"].view(np.int16)).view(torch.bfloat16).to(dev)
        wq, ws = mxfp8.quantize_weight(w0, "e4m3")
        pk = mxfp8.prepack_weight(wq, ws, "e4m3")
        bias = torch.from_numpy(dd["bias"].view(np.int16)).view(torch.bfloat16).to(dev)
        RD = 32
        # the stream floor: a plain read of the same weight bytes, 32 rotated copies, replayed
        # from a HIP graph exactly as the decode calls are
        floor_us = None
        if peaks_lib is not None:
            floor_us, fu, fb = stream_read_us(peaks_lib, pk.numel(), sets=RD)
            decode["stream_floor"] = {"bytes": pk.numel(), "us_per_read": round(floor_us, 3),
                                      "GB/s": round(pk.numel() / floor_us / 1e3, 1),
                                      "unroll": fu, "blocks": fb}
        pks = [pk] + [pk.clone() for _ in range(RD - 1)]
        for Md in (1, 8, 32, 64, 128):
            xd = torch.from_numpy(dd["x"][:Md].view(np.int16)).view(torch.bfloat16).to(dev)
            yd = torch.empty((Md, Nd), dtype=torch.bfloat16, device=dev)
            wsd = torch.zeros(max(1, mxfp8.workspace_bytes(Md, Nd, Kd)), dtype=torch.uint8, device=dev)
            s = torch.cuda.Stream(dev)
            s.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(s):
                for j in range(RD):                     # eager warm-up on the capture stream
                    mxfp8.linear(xd, pks[j], Nd, "e4m3", bias, out=yd, workspace=wsd)
            torch.cuda.current_stream(dev).wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for j in range(RD):
                    mxfp8.linear(xd, pks[j], Nd, "e4m3", bias, out=yd, workspace=wsd)
            reps = max(4, args.steps // 8)
            g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) * 1e6 / (reps * RD)
            bytes_alg = Md * Kd * 2 + (pk.numel()) + Md * Nd * 2 + Nd * 2
            gbs = bytes_alg / (us * 1e-6) / 1e9
            decode["M%d" % Md] = {
                "us_per_call": round(us, 3), "TFLOP/s": round(2.0 * Md * Nd * Kd / (us * 1e-6) / 1e12, 3),
                "algorithmic_bytes": bytes_alg, "GB/s": round(gbs, 1),
                "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                "hbm_frac_attainable": round(gbs / att_hbm, 4) if att_hbm else None,
                "x_stream_floor": round(us / floor_us, 3) if floor_us else None}
            # the same calls in batch-invariant mode (no split-K kernels)
            mxfp8.set_batch_invariant(True)
            try:
                with torch.cuda.stream(s):
                    for j in range(RD):
                        mxfp8.linear(xd, pks[j], Nd, "e4m3", bias, out=yd, workspace=wsd)
                torch.cuda.current_stream(dev).wait_stream(s)
                torch.cuda.synchronize()
                gi = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gi, stream=s):
                    for j in range(RD):
                        mxfp8.linear(xd, pks[j], Nd, "e4m3", bias, out=yd, workspace=wsd)
                gi.replay()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(reps):
                    gi.replay()
                torch.cuda.synchronize()
                decode["M%d" % Md]["batch_invariant_us_per_call"] = round(
                    (time.perf_counter() - t0) * 1e6 / (reps * RD), 3)
                del gi
            finally:
                mxfp8.set_batch_invariant(False)
            del g
        # the same decode layers eight at a time through the batched entry (B independent
        # layers, each with its own activations, weight and bias, in one launch), replayed from a
        # HIP graph over the same 32 rotated weights: the weight stream of one launch is then
        # 8 x 17.3 MB instead of 17.3 MB
        Bd, RB = 8, 64                         # 64 weights, 1.1 GB: no reuse from the caches
        pkb = [torch.cat([pks[(b * Bd + i) % RD] for i in range(Bd)]) for b in range(RB // Bd)]
        biasb = bias.unsqueeze(0).repeat(Bd, 1).contiguous()
        decode["batched8"] = {"layers_per_call": Bd, "rotated_weights": RB}
        for Md in (1, 8, 32):
            xb8 = torch.from_numpy(dd["x"][:Md].view(np.int16)).view(torch.bfloat16).to(dev)
            xb8 = xb8.unsqueeze(0).repeat(Bd, 1, 1).contiguous()
            yb8 = torch.empty((Bd, Md, Nd), dtype=torch.bfloat16, device=dev)
            wsd = torch.zeros(max(1, mxfp8.workspace_bytes(Bd * Md, Nd, Kd)), dtype=torch.uint8,
                              device=dev)
            s = torch.cuda.Stream(dev)
            s.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(s):
                for j in range(RB // Bd):
                    mxfp8.linear_batched(xb8, pkb[j], Nd, "e4m3", biasb, out=yb8, workspace=wsd)
            torch.cuda.current_stream(dev).wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for j in range(RB // Bd):
                    mxfp8.linear_batched(xb8, pkb[j], Nd, "e4m3", biasb, out=yb8, workspace=wsd)
            reps = max(4, args.steps // 2)
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) * 1e6 / (reps * RB)        # per layer
            bytes_alg = Md * Kd * 2 + pks[0].numel() + Md * Nd * 2 + Nd * 2
            gbs = bytes_alg / (us * 1e-6) / 1e9
            decode["batched8"]["M%d" % Md] = {
                "us_per_layer": round(us, 3), "GB/s": round(gbs, 1),
                "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                "hbm_frac_attainable": round(gbs / att_hbm, 4) if att_hbm else None,
                "x_stream_floor": round(us / floor_us, 3) if floor_us else None}
            del g, xb8, yb8, wsd
        del pkb, pks, pk

    # ------------------------------------------------------------ the other workloads
    others = None
    if not args.no_others:
        torch.cuda.empty_cache()
        others = {}

        def bf16_dev(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

        def rotated(make_set, set_bytes):
            n = max(2, -(-2 * MALL_BYTES // set_bytes))
            return [make_set(j) for j in range(n)]

        timing_detail = {}

        def time_calls(fn, n_sets, iters, name=None):
            """Calls of fn for --settle-ms / 2 of GPU time (every set touched; the chip reaches
            the steady clock of this workload: 100 calls were measured 15 % slow on the
            outlier GEMM), then 5 loops of `iters` calls timed with HIP events on the current
            stream: the median per call (the min goes to timing_detail[name])."""
            j = 0
            t_end = time.perf_counter() + args.settle_ms / 2e3
            while j < 2 * n_sets or time.perf_counter() < t_end:
                fn(j % n_sets)
                j += 1
                if j % 20 == 0:
                    torch.cuda.synchronize()
            torch.cuda.synchronize()
            stream = torch.cuda.current_stream(dev)
            per = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(iters):
                    fn(i % n_sets)
                e1.record(stream)
                torch.cuda.synchronize()
                per.append(e0.elapsed_time(e1) * 1e3 / iters)
            if name:
                timing_detail[name] = {"us_min": round(min(per), 2), "warm_calls": j}
            return statistics.median(per)

        # outlier activations on the pre-quantized entry (GEMM only), fused-QKV shape
        do = synth.make("outlier")
        Mo, No, Ko = do["M"], do["N"], do["K"]
        xq_o, xs_o = mxfp8.quantize_act(bf16_dev(do["x"]))
        wq, ws = mxfp8.quantize_weight(bf16_dev(do["w"]), "e4m3")
        pk_o = mxfp8.prepack_weight(wq, ws, "e4m3")
        del wq, ws
        sets = rotated(lambda j: (xq_o.clone(), xs_o.clone(), pk_o.clone(),
                                  torch.empty((Mo, No), dtype=torch.bfloat16, device=dev)),
                       xq_o.numel() + xs_o.numel() + pk_o.numel() + Mo * No * 2)
        us = time_calls(lambda j: mxfp8.linear_prequant(sets[j][0], sets[j][1], sets[j][2], No,
                                                        "e4m3", out=sets[j][3]),
                        len(sets), max(50, args.steps), "outlier")
        fl = 2.0 * Mo * No * Ko
        others["outlier_prequant_2048x6144x4096"] = {
            "us": round(us, 2), "TFLOP/s": round(fl / us / 1e6, 1),
            "mfma_frac": round(fl / us / 1e6 / PEAK_FP8_TFLOPS, 4), "rotated_sets": len(sets)}
        del sets, xq_o, xs_o, pk_o
        torch.cuda.empty_cache()

        # MXFP6 weights (E2M3, E3M2), bf16 activations quantized to MXFP8 inside the call
        dm = synth.make("mxfp6")
        Mf, Nf, Kf = dm["M"], dm["N"], dm["K"]
        xf = bf16_dev(dm["x"])
        wf = bf16_dev(dm["w"])
        for fname in ("e2m3", "e3m2"):
            wq, ws = mxfp8.quantize_weight(wf, fname)
            pk_f = mxfp8.prepack_weight(wq, ws, fname)
            del wq, ws
            sets = rotated(lambda j: (xf.clone(), pk_f.clone(),
                                      torch.empty((Mf, Nf), dtype=torch.bfloat16, device=dev)),
                           xf.numel() * 2 + pk_f.numel() + Mf * Nf * 2)
            wsf = torch.zeros(mxfp8.workspace_bytes(Mf, Nf, Kf, fname), dtype=torch.uint8, device=dev)
            us = time_calls(lambda j: mxfp8.linear(sets[j][0], sets[j][1], Nf, fname,
                                                   out=sets[j][2], workspace=wsf),
                            len(sets), max(50, args.steps), "mxfp6_" + fname)
            fl = 2.0 * Mf * Nf * Kf
            others["mxfp6_%s_512x8192x8192" % fname] = {
                "us": round(us, 2), "TFLOP/s": round(fl / us / 1e6, 1),
                "mfma_frac_fp8_rate": round(fl / us / 1e6 / PEAK_FP8_TFLOPS, 4),
                "rotated_sets": len(sets)}
            # the same weights with MXFP6 activations (same format as the weight): both MFMA
            # operands FP6, against the 10.1 PFLOP/s dense FP6 peak
            wsf6 = torch.zeros(mxfp8.workspace_bytes_fmt(Mf, Nf, Kf, fname, fname),
                               dtype=torch.uint8, device=dev)
            us6 = time_calls(lambda j: mxfp8.linear_fmt(sets[j][0], sets[j][1], Nf, fname, fname,
                                                        out=sets[j][2], workspace=wsf6),
                             len(sets), max(50, args.steps), "w6a6_" + fname)
            others["w6a6_%s_512x8192x8192" % fname] = {
                "us": round(us6, 2), "TFLOP/s": round(fl / us6 / 1e6, 1),
                "mfma_frac_fp6_rate": round(fl / us6 / 1e6 / PEAK_FP6_TFLOPS, 4),
                "rotated_sets": len(sets)}
            del sets, pk_f, wsf, wsf6
        del xf, wf
        torch.cuda.empty_cache()

        # fused producer: RMS norm + MXFP8 quantization of the prefill activations, against a
        # torch RMS norm followed by the standalone quantizer (same rotated buffers)
        Mp, Kp = 4096, 4096
        gp = torch.Generator(device=dev)
        gp.manual_seed(0)
        gam = (torch.rand(Kp, generator=gp, device=dev) + 0.5).to(torch.bfloat16)
        xp_bytes = Mp * Kp * 2
        sets = rotated(lambda j: (torch.randn((Mp, Kp), generator=gp, device=dev).to(torch.bfloat16),
                                  torch.empty((Mp, Kp), dtype=torch.uint8, device=dev),
                                  torch.empty((Mp, Kp // 32), dtype=torch.uint8, device=dev)),
                       xp_bytes + Mp * Kp + Mp * Kp // 32)
        L = mxfp8.lib()
        st = torch.cuda.current_stream(dev).cuda_stream

        def fused(j):
            x_, q_, s_ = sets[j]
            rc = L.mxfp8_rmsnorm_quantize_act(x_.data_ptr(), Mp, Kp, Kp, gam.data_ptr(), 1e-6,
                                              q_.data_ptr(), s_.data_ptr(), None, st)
            assert rc == 0, L.mxfp8_last_error()

        def separate(j):
            x_, q_, s_ = sets[j]
            yn = torch.nn.functional.rms_norm(x_, (Kp,), gam, 1e-6)
            rc = L.mxfp8_quantize_act(yn.data_ptr(), Mp, Kp, Kp, q_.data_ptr(), s_.data_ptr(), st)
            assert rc == 0, L.mxfp8_last_error()

        us_f = time_calls(fused, len(sets), max(50, args.steps), "producer")
        us_s = time_calls(separate, len(sets), max(50, args.steps), "producer_torch")
        alg = 3.03125 * Mp * Kp + 2 * Kp
        others["producer_rmsnorm_quant_4096x4096"] = {
            "us": round(us_f, 2), "GB/s": round(alg / us_f / 1e3, 1),
            "hbm_frac": round(alg / us_f / 1e3 / PEAK_HBM_GBS, 4),
            "us_torch_rms_norm_then_quantizer": round(us_s, 2), "rotated_sets": len(sets)}
        del sets, gam
        torch.cuda.empty_cache()

        # tiny: latency of one call (HIP graph of 64 calls)
        dt = synth.make("tiny")
        xt = bf16_dev(dt["x"])
        wq, ws = mxfp8.quantize_weight(bf16_dev(dt["w"]), "e4m3")
        pk_t = mxfp8.prepack_weight(wq, ws, "e4m3")
        yt = torch.empty((dt["M"], dt["N"]), dtype=torch.bfloat16, device=dev)
        wst = torch.zeros(max(1, mxfp8.workspace_bytes(dt["M"], dt["N"], dt["K"])), dtype=torch.uint8, device=dev)
        st = torch.cuda.Stream(dev)
        st.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(st):
            mxfp8.linear(xt, pk_t, dt["N"], "e4m3", out=yt, workspace=wst)
        torch.cuda.current_stream(dev).wait_stream(st)
        torch.cuda.synchronize()
        gt = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gt, stream=st):
            for _ in range(64):
                mxfp8.linear(xt, pk_t, dt["N"], "e4m3", out=yt, workspace=wst)
        gt.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(20):
            gt.replay()
        torch.cuda.synchronize()
        others["tiny_16x256x512_us_per_call"] = round((time.perf_counter() - t0) * 1e6 / (20 * 64), 3)
        del gt, xt, pk_t, yt, wst

        # batched layer: 8 independent 512 x 4096 x 4096 layers in one call vs 8 calls
        Bb, Mb, Nb, Kb = 8, 512, 4096, 4096
        gb = torch.Generator(device=dev)
        gb.manual_seed(0)
        xb = torch.randn((Bb, Mb, Kb), generator=gb, device=dev).to(torch.bfloat16)
        pks = []
        for _ in range(Bb):
            wq, ws = mxfp8.quantize_weight(
                (torch.randn((Nb, Kb), generator=gb, device=dev) * 0.02).to(torch.bfloat16), "e4m3")
            pks.append(mxfp8.prepack_weight(wq, ws, "e4m3"))
        pkb = torch.cat(pks)
        del pks, wq, ws
        yb = torch.empty((Bb, Mb, Nb), dtype=torch.bfloat16, device=dev)
        wsb2 = torch.zeros(max(mxfp8.workspace_bytes(Bb * Mb, Nb, Kb), mxfp8.workspace_bytes(Mb, Nb, Kb)),
                           dtype=torch.uint8, device=dev)   # batched call and single calls
        P = mxfp8.prepacked_bytes(Nb, Kb)
        us_b = time_calls(lambda j: mxfp8.linear_batched(xb, pkb, Nb, "e4m3", out=yb, workspace=wsb2),
                          1, max(20, args.steps // 4), "batched")
        us_s = time_calls(lambda j: [mxfp8.linear(xb[b], pkb[b * P:(b + 1) * P], Nb, "e4m3",
                                                  out=yb[b], workspace=wsb2) for b in range(Bb)],
                          1, max(20, args.steps // 4), "batched_separate")
        fl = 2.0 * Bb * Mb * Nb * Kb
        others["batched_8x512x4096x4096"] = {
            "us": round(us_b, 2), "TFLOP/s": round(fl / us_b / 1e6, 1),
            "us_as_8_separate_calls": round(us_s, 2)}
        others["timing"] = {"protocol": "calls for --settle-ms / 2 of GPU time, then the median "
                                        "of 5 loops timed with HIP events (min below)",
                            "detail": timing_detail}
        del xb, pkb, yb, wsb2

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline and int(os.environ.get("RANK", "0")) == 0:
        def cpu_run(part, seconds, threads=None):
            env = dict(os.environ)
            env.pop("CUDA_VISIBLE_DEVICES", None)
            if threads:
                env["OMP_NUM_THREADS"] = str(threads)
            r = subprocess.run([sys.executable, "-m", "oracle.cpu_bench", "--workload", "prefill",
                                "--part", part, "--seconds", str(seconds)],
                               cwd=ROOT, capture_output=True, text=True, env=env)
            if r.returncode != 0:
                return {"error": r.stderr[-300:]}
            return json.loads(r.stdout.strip().splitlines()[-1])

        c = cpu_run("layer", args.cpu_seconds)
        if "error" in c:
            cpu = c
        else:
            cpu = {"value": c["value"], "unit": c["unit"], "cores": c["cores"],
                   "kind": "oracle", "sample": c["sample"], "cpu_model": c.get("cpu_model")}
            part_s = max(1.0, args.cpu_seconds / 4)
            for part, key in (("quant", "quantizer"), ("gemm", "fp64_gemm")):
                for th, tag in ((None, "all_cores"), (1, "one_thread")):
                    r = cpu_run(part, part_s, th)
                    cpu["%s_%s" % (key, tag)] = (
                        r if "error" in r else {"value": round(r["value"], 3), "unit": r["unit"],
                                                "cores": r["cores"], "sample": r["sample"]})

    out = {
        "metric": "MXFP8 linear TFLOP/s (incl. act quant) and % MFMA/HBM roofline, prefill & decode",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8-e4m3 (mxfp8) -> fp32 acc -> bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights quantized on the GPU)",
        "config": {"workload": "prefill MLP up-proj: x bf16 [4096,4096] x W mxfp8 [14336,4096] "
                               "-> y bf16 [4096,14336], act quant included",
                   "M": M, "N": N, "K": K, "rotated_sets": R, "inputs_sha256_16": inputs_sha},
        "roofline": roofline,
        "quantizer": quantizer,
        "step_protocol": step_protocol,
        "clock": clock,
        "attainable": attainable,
        "decode": decode,
        "other_workloads": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
