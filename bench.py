#!/usr/bin/env python3
"""Benchmark of the weight-only quantized skinny GEMM on one MI355X.

Metric: effective weight-read bandwidth in GB/s, i.e. compressed weight bytes
(E2M1 codes + E4M3 scales + the 4-byte global scale; FP8: codes + fp32 block
scales) per step divided by the time per step, with every input already
resident in HBM.  The headline workload is the NVFP4 GEMV at M = 1,
K = 5120, N = 17408 (an MLP up-projection at decode): one step is one
nvfp4_gemm call.  The same line also carries, timed the same way:
  * the NVFP4 M = 8 shapes: fused gate+up 5120 x 34816, down 17408 x 5120,
    and gate+up with the fused SwiGLU epilogue (nvfp4_gemm_swiglu, h[8, 17408]);
  * the other two NVFP4 MLP projections at M = 1: gate+up and down;
  * the FP8 shapes qkv 5120 x 7168 and o_proj 6144 x 5120 at M = 1, 2 and 4,
    with canonical codes (fp8_gemm) and packed codes (fp8_gemm_packed);
  * the 151936-column NVFP4 lm_head with its fused argmax at M = 1 and 8;
  * one decoder block's four GEMMs in the published FP8/FP4 mix
    (skinny_layers_run) at M = 8.
Each shape reports the measured read ceiling at its weight size: the
library's read probe (skinny_read_probe, one 9 KiB block per single-wavefront
workgroup, the fastest pattern of the read sweep) over the same rotating
copies; the headline adds the probe over a 2 GiB buffer.

    python bench.py [--steps K] [--warmup W] [--workload up|gate_up|down|qkv|o_proj|lm_head|gate_up_swiglu|lm_head_verify|block|qkv_packed|o_proj_packed] [--M m]
    python bench.py --read-sweep [--workload up]     every read pattern of skinny_read_probe_pattern

Each step reads a different one of R byte-identical copies of the weights
(R copies exceed 600 MB) so that the 256 MB Infinity Cache cannot serve them.
Timing: W eager warm-up steps, then the K steps are captured once into a HIP
graph, which is replayed untimed for about 0.1 s (GPU clocks settle only
after tens of milliseconds of work); the timed region is one more replay,
bracketed by device synchronisation, with a HIP event pair recorded on the
replay stream.  The kernels of a replay run back to back, so the per-launch
kernel duration is the event time divided by K.  Six more replays, timed the
same way after the timed region, give the spread (p10 / median / p90 of the
per-step time over the seven replays).  The CPU oracle is timed beside it on
the host, on a bounded sample of the headline workload.
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
CPU_BASELINE_SECONDS = 10.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="up")
    ap.add_argument("--M", type=int, default=None, help="row count (default: the workload's largest)")
    ap.add_argument("--config", default=None, help="explicit kernel choice engine,ct,nw,ksplit")
    ap.add_argument("--headline-only", action="store_true", help="skip the M = 8 companion shapes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--read-sweep", action="store_true",
                    help="only time every read pattern of skinny_read_probe_pattern at the workload's weight size")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run five device-to-device copies of MB megabytes (the known-size "
                         "kernel that scales the HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {time.strftime('%H:%M:%S')} {msg}", file=sys.stderr, flush=True)


def describe(case, name):
    if name.endswith("_packed"):
        return f"FP8 E4M3 W8A16 {name} M={case['M']} K={case['K']} N={case['N']} (codes packed by fp8_pack)"
    if case["fmt"] == "swiglu":
        return f"NVFP4 W4A16 {name} M={case['M']} K={case['K']} F={case['F']} (gate and up, h = silu(gate) * up)"
    fmt = "NVFP4 W4A16" if case["fmt"] == "nvfp4" else "FP8 E4M3 W8A16"
    extra = (" + fused argmax" if name == "lm_head" else
             " + fused argmax and greedy verification of 7 drafts" if name == "lm_head_verify" else "")
    return f"{fmt} {name} M={case['M']} K={case['K']} N={case['N']}{extra}"


def cpu_baseline(case):
    """Time the CPU oracle on the whole headline workload, repeated for about 10 s."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    calls, t0 = 0, time.perf_counter()
    while True:
        if case["fmt"] == "nvfp4":
            oracle.nvfp4_gemm(case["x"], case["codes"], case["scales"], case["g"])
        else:
            oracle.fp8_gemm(case["x"], case["codes"], case["scales"])
        calls += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_BASELINE_SECONDS:
            break
    gbs = case["weight_bytes"] * calls / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": blas_threads, "kind": "oracle",
            "sample": f"the whole workload ({case['N']} columns), {calls} calls in {dt:.1f} s; "
                      f"decode and dequantize on 1 thread, float64 matmul on {blas_threads} BLAS "
                      f"threads; host has {os.cpu_count()} CPUs, {len(os.sched_getaffinity(0))} "
                      f"usable by this process ({cpu_model()})"}


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo, or "unknown CPU"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.partition(":")[2].strip()
    except OSError:
        pass
    return "unknown CPU"


def recorded_traffic(name, M):
    """HBM bytes per launch from a committed counter summary under profiles/.

    Used only if that summary was taken on the current kernel sources (same
    SHA-256) for this workload; otherwise None."""
    import glob
    from fp8_quantized_skinny_amd.profile_summary import sources_sha256
    sha = sources_sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt"))):
        fields = {}
        with open(path) as f:
            for line in f:
                key, sep, val = line.partition(":")
                if sep and key.strip() and " " not in key.strip():
                    fields.setdefault(key.strip(), val.strip())
        if (fields.get("workload") == f"{name} M={M}" and fields.get("kernel_sources_sha256") == sha
                and "traffic_bytes_per_launch" in fields):
            return int(fields["traffic_bytes_per_launch"].split()[0])
    return None


def time_graph(step, steps, stream, extra=0):
    """Capture `steps` launches of step(i, stream_handle) in a HIP graph, replay it untimed for
    about 0.1 s (clocks and power state settle only after tens of milliseconds of back-to-back
    kernels), then time one replay with HIP events on `stream` (the timed region).  `extra` more
    replays are timed the same way afterwards, for the spread.  Returns (ms of the timed replay,
    [ms of each extra replay])."""
    import torch
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(steps):
                step(i, torch.cuda.current_stream().cuda_stream)
    t_warm = time.perf_counter()
    for _ in range(50):
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t_warm > 0.1:
            break
    times = []
    for _ in range(1 + extra):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del g
    return times[0], times[1:]


def spread(us_list):
    """p10 / median / p90 of per-step times (us) over graph replays."""
    import numpy as np
    a = np.asarray(us_list, dtype=np.float64)
    return {"replays": int(a.size), "us_p10": round(float(np.percentile(a, 10)), 3),
            "us_median": round(float(np.median(a)), 3), "us_p90": round(float(np.percentile(a, 90)), 3)}


def probe_size(nbytes, buffers):
    """Bytes the read probe reads from each buffer: the weight bytes rounded down
    to whole 9216-byte blocks, never more than the smallest buffer holds (FP8
    weight bytes count the block scales, which live outside the code buffers)."""
    cap = min(b.numel() * b.element_size() for b in buffers)
    size = (min(int(nbytes), cap) // 9216) * 9216
    if size < 9216 or size > cap:
        raise ValueError(f"read probe of {size} bytes does not fit buffers of {cap} bytes")
    return size


def read_ceiling(copies, nbytes, steps, large=True):
    """Measured HBM read ceiling: the library's read probe (one 9 KiB block per
    wavefront, nine 16-byte loads per lane) over the same rotating copies as the
    GEMM, and over a 2 GiB buffer."""
    import torch
    import fp8_quantized_skinny_amd as sk
    from fp8_quantized_skinny_amd._lib import lib
    L = lib()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    probe_bytes = probe_size(nbytes, copies)

    def step_same(i, s):
        st = L.skinny_read_probe(copies[i % len(copies)].data_ptr(), probe_bytes, sink.data_ptr(), s)
        if st != 0:
            raise RuntimeError(f"read probe failed: {sk.strerror(st)}")
    ms, _ = time_graph(step_same, steps, stream)
    same = probe_bytes * steps / (ms * 1e-3) / 1e9
    out = {"same_size_GBs": round(same, 1),
           "probe": "skinny_read_probe: one 9 KiB block per single-wavefront workgroup, nine 16-byte "
                    "non-temporal loads per lane (the fastest read pattern of bench.py --read-sweep); "
                    "same rotation of weight copies as the GEMM, HIP-graph replay"}
    log(f"read probe: {same:.1f} GB/s at {nbytes / 1e6:.1f} MB")
    if not large:
        return out
    big = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    big_bytes = probe_size(big.numel(), [big])

    def step_big(i, s):
        st = L.skinny_read_probe(big.data_ptr(), big_bytes, sink.data_ptr(), s)
        if st != 0:
            raise RuntimeError(f"read probe failed: {sk.strerror(st)}")
    ms_big, _ = time_graph(step_big, 20, stream)
    large_gbs = big_bytes * 20 / (ms_big * 1e-3) / 1e9
    del big
    log(f"read probe: {large_gbs:.1f} GB/s at 2 GiB")
    out["2GiB_GBs"] = round(large_gbs, 1)
    return out


def prepare(name, M=None):
    """The host case of a workload (seeded draw, library quantizer, packed blob) at its largest M."""
    from fp8_quantized_skinny_amd import workload, synth
    fmt, ms, K, N = synth.WORKLOADS[name]
    M = M or max(ms)
    t = time.perf_counter()
    case = (workload.nvfp4_case(M, K, N) if fmt == "nvfp4" else
            workload.swiglu_case(M, K, N) if fmt == "swiglu" else workload.fp8_case(M, K, N))
    log(f"prepared {name} (M up to {M}, K={K}, N={N}) in {time.perf_counter() - t:.1f} s")
    return case


def measure(name, M, cfg, steps, warmup, case=None, ceiling=False, large_probe=False, extra=6):
    """Time `steps` launches of one workload at M rows; returns the result dict.

    case: a prepared case of the same workload with at least M rows of x (its
    leading M rows are used; the weights do not depend on M)."""
    import numpy as np
    import torch
    import fp8_quantized_skinny_amd as sk
    from fp8_quantized_skinny_amd import synth
    from fp8_quantized_skinny_amd._lib import lib

    fmt, ms, K, N = synth.WORKLOADS[name]
    M = M or max(ms)
    case = case if case is not None else prepare(name, M)
    assert case["x"].shape[0] >= M
    packed = fmt == "fp8p"
    wbytes = case["weight_bytes"]
    R = max(2, math.ceil(MIN_ROTATION_BYTES / wbytes))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    L = lib()
    x = dev(case["x"][:M])
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    idx = torch.empty((M,), dtype=torch.int32, device="cuda")
    if fmt in ("nvfp4", "swiglu"):
        copies = [dev(case["blob"]) for _ in range(R)]
        scales = None
    else:
        codes = sk.fp8_pack(case["codes"], K, N) if packed else case["codes"]
        copies = [dev(codes) for _ in range(R)]
        scales = dev(case["scales"])
    verify = name == "lm_head_verify"
    op = (sk.OP_LM_HEAD if name in ("lm_head", "lm_head_verify") else sk.OP_SWIGLU if fmt == "swiglu" else
          sk.OP_NVFP4 if fmt == "nvfp4" else sk.OP_FP8)
    drafts = torch.zeros((max(M - 1, 1),), dtype=torch.int32, device="cuda")
    result = torch.empty((M + 1,), dtype=torch.int32, device="cuda")
    ws = torch.zeros(max(sk.workspace_bytes(op, M, K, N, cfg), 256), dtype=torch.uint8, device="cuda")
    wsp, wsn = ws.data_ptr(), ws.numel()
    xp, yp = x.data_ptr(), y.data_ptr()

    def step(i, s):
        w = copies[i % R].data_ptr()
        if verify:
            st = (L.lm_head_verify_greedy_config(w, xp, drafts.data_ptr(), idx.data_ptr(), result.data_ptr(),
                                                 M, K, N, wsp, wsn, s, *cfg) if cfg
                  else L.lm_head_verify_greedy(w, xp, drafts.data_ptr(), idx.data_ptr(), result.data_ptr(),
                                               M, K, N, wsp, wsn, s))
        elif op == sk.OP_LM_HEAD:
            st = (L.lm_head_gemm_argmax_config(w, xp, idx.data_ptr(), None, M, K, N, wsp, wsn, s, *cfg) if cfg
                  else L.lm_head_gemm_argmax(w, xp, idx.data_ptr(), None, M, K, N, wsp, wsn, s))
        elif op == sk.OP_NVFP4:
            st = (L.nvfp4_gemm_config(w, xp, yp, M, K, N, wsp, wsn, s, *cfg) if cfg
                  else L.nvfp4_gemm(w, xp, yp, M, K, N, wsp, wsn, s))
        elif op == sk.OP_SWIGLU:   # N is F here; y holds h[M, F]
            st = (L.nvfp4_gemm_swiglu_config(w, xp, yp, M, K, N, wsp, wsn, s, *cfg) if cfg
                  else L.nvfp4_gemm_swiglu(w, xp, yp, M, K, N, wsp, wsn, s))
        elif packed:
            st = (L.fp8_gemm_packed_config(w, scales.data_ptr(), xp, yp, M, K, N, wsp, wsn, s, *cfg) if cfg
                  else L.fp8_gemm_packed(w, scales.data_ptr(), xp, yp, M, K, N, wsp, wsn, s))
        else:
            st = (L.fp8_gemm_config(w, scales.data_ptr(), xp, yp, M, K, N, wsp, wsn, s, *cfg) if cfg
                  else L.fp8_gemm(w, scales.data_ptr(), xp, yp, M, K, N, wsp, wsn, s))
        if st != 0:
            raise RuntimeError(f"launch failed: {sk.strerror(st)}")

    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i, stream.cuda_stream)
    torch.cuda.synchronize()

    # Timed region: one replay of the K-step graph on `stream`, after untimed replays.
    gpu_ms, more = time_graph(step, steps, stream, extra=extra)
    log(f"{name} M={M}: graph replay {gpu_ms:.3f} ms GPU for {steps} steps")
    us = gpu_ms * 1e3 / steps
    gbs = wbytes / (us * 1e-6) / 1e9
    res = {"workload": describe(dict(case, M=M), name), "M": M, "K": K, "N": N, "weight_bytes": wbytes,
           "weight_copies": R, "kernel_choice": list(cfg) if cfg else list(sk.default_config(op, M, K, N)),
           "us_per_step": round(us, 3), "GB/s": round(gbs, 2), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    if extra:
        res["spread"] = spread([t * 1e3 / steps for t in [gpu_ms] + more])
    if ceiling:
        res["read_ceiling"] = read_ceiling(copies, wbytes, steps, large=large_probe)
        res["frac_of_read_ceiling"] = round(gbs / res["read_ceiling"]["same_size_GBs"], 4)
    del copies
    torch.cuda.synchronize()
    return res


def read_sweep(name, steps):
    """HBM read rate of each read pattern of skinny_read_probe_pattern at the workload's weight size,
    over the same rotation of copies as the GEMM (bench.py --read-sweep)."""
    import ctypes
    import torch
    import fp8_quantized_skinny_amd as sk
    from fp8_quantized_skinny_amd import synth
    from fp8_quantized_skinny_amd._lib import lib
    L = lib()
    fmt, ms, K, N = synth.WORKLOADS[name]
    ku, nt = -(-K // 1024), -(-N // 16)
    nbytes = ku * nt * 9216 if fmt == "nvfp4" else K * N
    R = max(2, math.ceil(MIN_ROTATION_BYTES / nbytes))
    copies = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    patterns = [("blocks 9 KiB, 1 wavefront per workgroup (skinny_read_probe)", 0, 1, 0),
                ("blocks 9 KiB, 2 wavefronts per workgroup", 0, 2, 0),
                ("blocks 9 KiB, 4 wavefronts per workgroup", 0, 4, 0),
                ("blocks 9 KiB, 8 wavefronts per workgroup", 0, 8, 0),
                ("blocks 9 KiB, 16 wavefronts per workgroup", 0, 16, 0),
                ("blocks 4 KiB, 4 wavefronts per workgroup", 1, 4, 0),
                ("blocks 18 KiB, 2 wavefronts per workgroup", 2, 2, 0),
                ("blocks 18 KiB, 4 wavefronts per workgroup", 2, 4, 0),
                (f"tiles of {ku} spans, one workgroup per tile (the NVFP4 GEMV's shape)", 3, ku, 0),
                ("persistent, 256 workgroups x 4 wavefronts, 2 blocks in flight", 4, 256, 4),
                ("persistent, 256 workgroups x 8 wavefronts, 2 blocks in flight", 4, 256, 8),
                ("persistent, 1024 workgroups x 4 wavefronts, 2 blocks in flight", 4, 1024, 4)]
    for flight, pat in ((3, 5), (4, 6)):  # wavefronts per SIMD 1, 2, 4, 8 and 1, 2, 4 workgroups per CU
        for groups, waves in ((256, 4), (256, 8), (256, 16), (512, 8), (1024, 4), (1024, 8)):
            patterns.append((f"persistent, {groups} workgroups x {waves} wavefronts, {flight} blocks in flight",
                             pat, groups, waves))
    out = []
    for label, pattern, a, b in patterns:
        if pattern == 3 and not 1 <= a <= 16:
            continue
        got = ctypes.c_size_t(0)

        def step(i, s, pattern=pattern, a=a, b=b, got=got):
            st = L.skinny_read_probe_pattern(copies[i % R].data_ptr(), nbytes, pattern, a, b, sink.data_ptr(),
                                             ctypes.byref(got), s)
            if st != 0:
                raise RuntimeError(f"read probe failed: {sk.strerror(st)}")
        ms_, more = time_graph(step, steps, stream, extra=4)
        per = [t * 1e3 / steps for t in [ms_] + more]
        us = sorted(per)[len(per) // 2]
        out.append({"pattern": label, "bytes": got.value, "us_median": round(us, 3),
                    "GB/s": round(got.value / (us * 1e-6) / 1e9, 1)})
        log(f"read sweep {label}: {us:.3f} us, {out[-1]['GB/s']} GB/s")
    del copies
    return {"workload": name, "weight_bytes_per_copy": nbytes, "copies": R, "patterns": out}


def measure_block(M, steps, warmup):
    """One decoder block's GEMMs in the published mixed allocation, through one
    layer-table call per step: qkv and o_proj in FP8 (codes packed by
    fp8_pack), gate+up (SwiGLU pair) and down in NVFP4.  Each layer reads a
    different one of R copies per step."""
    import numpy as np
    import torch
    import fp8_quantized_skinny_amd as sk
    from fp8_quantized_skinny_amd import workload, synth

    t = time.perf_counter()
    _, _, Kq, Nq = synth.WORKLOADS["qkv"]
    _, _, Ko, No = synth.WORKLOADS["o_proj"]
    _, _, Kg, F = synth.WORKLOADS["gate_up_swiglu"]
    _, _, Kd, Nd = synth.WORKLOADS["down"]
    qkv, o = workload.fp8_case(M, Kq, Nq), workload.fp8_case(M, Ko, No)
    gu, dn = workload.swiglu_case(M, Kg, F), workload.nvfp4_case(M, Kd, Nd)
    wbytes = sum(c["weight_bytes"] for c in (qkv, o, gu, dn))
    log(f"prepared the block (4 layers, {wbytes / 1e6:.1f} MB) in {time.perf_counter() - t:.1f} s")
    R = max(2, math.ceil(MIN_ROTATION_BYTES / wbytes))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    qkv_p, o_p = sk.fp8_pack(qkv["codes"], Kq, Nq), sk.fp8_pack(o["codes"], Ko, No)
    tables = []
    for _ in range(R):
        tables.append([(sk.LAYER_FP8_PACKED, dev(qkv_p), dev(qkv["scales"]), Kq, Nq),
                       (sk.LAYER_FP8_PACKED, dev(o_p), dev(o["scales"]), Ko, No),
                       (sk.LAYER_SWIGLU, dev(gu["blob"]), None, Kg, F),
                       (sk.LAYER_NVFP4, dev(dn["blob"]), None, Kd, Nd)])
    xs = [dev(c["x"]) for c in (qkv, o, gu, dn)]
    ys = [torch.empty((M, n), dtype=torch.float16, device="cuda") for n in (Nq, No, F, Nd)]
    n = sk.layers_workspace_bytes(tables[0], M)
    ws = torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i, s):
        sk.layers_run(tables[i % R], xs, ys, workspace=ws, stream=s)
    for i in range(warmup):
        step(i, stream.cuda_stream)
    torch.cuda.synchronize()
    gpu_ms, more = time_graph(step, steps, stream, extra=6)
    us = gpu_ms * 1e3 / steps
    gbs = wbytes / (us * 1e-6) / 1e9
    log(f"block M={M}: {us:.2f} us per step")
    return {"workload": f"decoder block M={M}: qkv FP8 {Kq}x{Nq}, o_proj FP8 {Ko}x{No} (packed), "
                        f"gate+up NVFP4 SwiGLU {Kg}x2x{F}, down NVFP4 {Kd}x{Nd}",
            "M": M, "weight_bytes": wbytes, "weight_copies": R, "us_per_step": round(us, 3),
            "GB/s": round(gbs, 2), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "spread": spread([t * 1e3 / steps for t in [gpu_ms] + more])}


def companions(steps, warmup):
    """The other configurations of the benchmark, timed like the headline: the NVFP4 M = 8
    shapes, the other two NVFP4 MLP projections at M = 1, the FP8 shapes at M = 1, 2, 4
    (canonical and packed codes) and the lm_head at M = 1 and 8, each with the read ceiling at
    its weight size."""
    m8 = []
    for name in ("gate_up", "down", "gate_up_swiglu"):
        m8.append(measure(name, 8, None, steps, warmup, ceiling=name != "gate_up_swiglu"))
    m1 = [measure(name, 1, None, steps, warmup) for name in ("gate_up", "down")]
    fp8 = []
    for name in ("qkv", "o_proj"):
        case = prepare(name)
        for M in (1, 2, 4):
            for variant in (name, name + "_packed"):
                fp8.append(measure(variant, M, None, steps, warmup, case=case,
                                   ceiling=(M == 1 and variant == name)))
        del case
    lm = []
    case = prepare("lm_head")
    for M in (1, 8):
        lm.append(measure("lm_head", M, None, max(20, steps // 10), max(2, warmup // 10), case=case,
                          ceiling=M == 1))
    del case
    return m8, m1, fp8, lm


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the kernels have no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        import torch
        nbytes = args.copy_calibration * 1000 * 1000
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes, "copies": 5}), flush=True)
        return
    if args.read_sweep:
        print(json.dumps({"read_sweep": read_sweep(args.workload, args.steps)}), flush=True)
        return
    if args.workload == "block":
        res = measure_block(args.M or 8, args.steps, args.warmup)
        print(json.dumps({"metric": METRIC, "value": res["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
                          "warmup": args.warmup, "ms_per_step": round(res["us_per_step"] * 1e-3, 6),
                          "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
                          "data": "synthetic", "config": res}), flush=True)
        return
    cfg = tuple(int(v) for v in args.config.split(",")) if args.config else None
    case = prepare(args.workload, args.M)
    head = measure(args.workload, args.M, cfg, args.steps, args.warmup, case=case,
                   ceiling=not args.headline_only, large_probe=True)
    m8, m1, fp8, lm, block = [], [], [], [], None
    if not args.headline_only and args.workload == "up" and cfg is None:
        m8, m1, fp8, lm = companions(args.steps, args.warmup)
        block = measure_block(8, args.steps, args.warmup)
    value = head["GB/s"]
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] * 1e-3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {**head, "timed": "one HIP-graph replay of K steps, weights rotated over R copies; "
                                    "spread: that replay and 6 more",
                   "m8_shapes": m8, "m1_shapes": m1, "fp8_shapes": fp8, "lm_head_shapes": lm,
                   "decoder_block_m8": block},
        "roofline": {"bound": "hbm", "achieved": value, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4),
                     "traffic": None if cfg else recorded_traffic(args.workload, head["M"]),
                     "kernel_us": head["us_per_step"]},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(dict(case, x=case["x"][:head["M"]]))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
