#!/usr/bin/env python3
"""Benchmark of the weight-only quantized skinny GEMM on one MI355X.

Metric: effective weight-read bandwidth in GB/s, i.e. compressed weight bytes
(codes + scales + the 4-byte global scale) per step divided by the time per
step, with every input already resident in HBM.  The headline workload is the
NVFP4 GEMV at M = 1, K = 5120, N = 17408 (an MLP up-projection at decode);
one step is one nvfp4_gemm call.  Each step reads a different one of R
byte-identical copies of the packed weights (R copies exceed 512 MB) so that
the 256 MB Infinity Cache cannot serve them.

    python bench.py [--steps K] [--warmup W] [--workload up|gate_up|down|qkv|o_proj|lm_head]

Timing: W eager warm-up steps, then the K steps are captured once into a HIP
graph and the timed region is one replay of that graph, bracketed by device
synchronisation.  A second pass launches the same K steps eagerly with a HIP
event pair around each launch on the launch stream; the mean of those
durations is the kernel duration used for the roofline figure.
The CPU oracle is timed on a bounded sample of the same workload on the host.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "effective weight-read GB/s (% of MI355X HBM peak), NVFP4 GEMM at M=1 and M=8"
MIN_ROTATION_BYTES = 600e6


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="up")
    ap.add_argument("--M", type=int, default=None, help="row count (default: the workload's largest)")
    ap.add_argument("--config", default=None, help="explicit kernel choice engine,ct,nw")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-cols", type=int, default=None)
    return ap.parse_args()


def describe(case, name):
    fmt = "NVFP4 W4A16" if case["fmt"] == "nvfp4" else "FP8 E4M3 W8A16"
    return f"{fmt} {name} M={case['M']} K={case['K']} N={case['N']}"


def cpu_baseline(case, sample_cols):
    """Time the CPU oracle on a bounded column sample; GB/s of weight bytes it covers."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    N = case["N"]
    cols = np.arange(min(sample_cols, N))
    frac = len(cols) / N
    t0 = time.perf_counter()
    if case["fmt"] == "nvfp4":
        oracle.nvfp4_gemm(case["x"], case["codes"], case["scales"], case["g"], cols=cols)
    else:
        oracle.fp8_gemm(case["x"], case["codes"], case["scales"], cols=cols)
    dt = time.perf_counter() - t0
    gbs = case["weight_bytes"] * frac / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": blas_threads, "kind": "oracle",
            "sample": f"first {len(cols)} of {N} columns ({frac:.3%} of the weights), one call, {dt:.1f} s; "
                      f"decode+dequant on 1 thread, float64 matmul on {blas_threads} BLAS threads; "
                      f"host has {os.cpu_count()} CPUs"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import fp8_quantized_skinny_amd as sk
    from fp8_quantized_skinny_amd import workload, synth
    from fp8_quantized_skinny_amd._lib import lib

    name = args.workload
    fmt, ms, K, N = synth.WORKLOADS[name]
    M = args.M or max(ms)
    t_prep = time.perf_counter()
    case = workload.nvfp4_case(M, K, N) if fmt == "nvfp4" else workload.fp8_case(M, K, N)
    print(f"[bench] prepared {describe(case, name)} in {time.perf_counter() - t_prep:.1f} s", file=sys.stderr,
          flush=True)
    wbytes = case["weight_bytes"]
    R = max(2, math.ceil(MIN_ROTATION_BYTES / wbytes))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    L = lib()
    x = dev(case["x"])
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    cfg = tuple(int(v) for v in args.config.split(",")) if args.config else None
    if fmt == "nvfp4":
        copies = [dev(case["blob"]) for _ in range(R)]
        scales = None
    else:
        copies = [dev(case["codes"]) for _ in range(R)]
        scales = dev(case["scales"])
    idx = torch.empty((M,), dtype=torch.int32, device="cuda")
    ws = torch.zeros(max(sk.workspace_bytes(sk.OP_LM_HEAD, M, K, N), 256), dtype=torch.uint8, device="cuda")

    def step(i, stream):
        w = copies[i % R].data_ptr()
        if name == "lm_head":
            if cfg:
                st = L.lm_head_gemm_argmax_config(w, x.data_ptr(), idx.data_ptr(), None, M, K, N, ws.data_ptr(),
                                                  ws.numel(), stream, *cfg)
            else:
                st = L.lm_head_gemm_argmax(w, x.data_ptr(), idx.data_ptr(), None, M, K, N, ws.data_ptr(),
                                           ws.numel(), stream)
        elif fmt == "nvfp4":
            st = (L.nvfp4_gemm_config(w, x.data_ptr(), y.data_ptr(), M, K, N, None, 0, stream, *cfg) if cfg
                  else L.nvfp4_gemm(w, x.data_ptr(), y.data_ptr(), M, K, N, None, 0, stream))
        else:
            st = (L.fp8_gemm_config(w, scales.data_ptr(), x.data_ptr(), y.data_ptr(), M, K, N, None, 0, stream, *cfg)
                  if cfg else L.fp8_gemm(w, scales.data_ptr(), x.data_ptr(), y.data_ptr(), M, K, N, None, 0, stream))
        if st != 0:
            raise RuntimeError(f"launch failed: {sk.strerror(st)}")

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        step(i, stream.cuda_stream)
    torch.cuda.synchronize()

    # Timed region: one replay of a graph holding exactly K steps.
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(args.steps):
                step(i, torch.cuda.current_stream().cuda_stream)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = gpu_ms / args.steps
    value = wbytes * args.steps / (gpu_ms * 1e-3) / 1e9

    # Per-launch kernel durations (event pair around each launch, same stream).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(i, stream.cuda_stream)
        b.record(stream)
    torch.cuda.synchronize()
    durs = np.array([a.elapsed_time(b) for a, b in evs])
    kern_ms = float(durs.mean())
    achieved = wbytes / (kern_ms * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": describe(case, name), "M": M, "K": K, "N": N, "weight_bytes": wbytes,
                   "weight_copies": R, "kernel_choice": list(cfg) if cfg else "default",
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4), "timed": "one HIP-graph replay of K steps"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel_us_mean": round(kern_ms * 1e3, 3), "kernel_us_p50": round(float(np.median(durs)) * 1e3, 3)},
    }
    print(f"[bench] graph replay: {gpu_ms:.3f} ms GPU, {wall * 1e3:.3f} ms wall for {args.steps} steps",
          file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        cols = args.cpu_sample_cols or max(256, min(N, int(N * 0.25)))
        out["cpu_baseline"] = cpu_baseline(case, cols)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
