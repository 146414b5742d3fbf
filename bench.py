#!/usr/bin/env python3
"""Throughput of the W4A16 dequantise-GEMM  C = A . dequant(B)^T  on one MI355X.

Default workload (the M = 1 weight-bandwidth case): decode GEMV with int4
asymmetric group-128 weights, M = 1, N = 8192, K = 3072, bf16 output.  One
step = one w4a16_gemm call.  `value` = weight GB/s = (packed + scales +
zeros bytes) per step / time per step, inputs resident in HBM.  The weights
rotate over enough distinct copies (>= 1 GiB) that no step finds them in the
256 MB last-level cache.  The same line carries the other workloads of the
metric, each with its own roofline fraction: the tiny int4 GEMM (M = 16), the
NVFP4 M = 16 GEMM, the compute-bound MXFP4 M = 4096 GEMM (TFLOP/s) and the
197-GEMV decode chain of a 3B decoder.

Timing.  The K timed steps are captured into one HIP graph (a decode step is
graph-captured in serving) and replayed once between two HIP events on the
launch stream, after a warm-up of the W requested steps and whole passes over
every rotating weight copy (first touch of each copy, clock ramp), a replay,
and about 1 ms of untimed replays queued behind a queue-fill spin (the spin
idles the GPU).  `ms_per_step` = the replay's time / K, and the roofline's
`achieved` uses the same mean duration per launch.  The same K steps are also
timed as eager launches (a spin kernel first fills the stream so that they run
back to back; from 500 steps on, the events split them into 5 repeats whose
median is reported) and reported as eager_ms_per_step.  The decode chain is
one batched call per step, timed the same way, with its layer-grouped and
single-launch forms beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Inputs are synthetic (seeded numpy draws: A ~ N(0, 1) in bf16, uniform codes,
scales / zeros drawn as the workload states).  The CPU baseline is the plain
fp64 oracle on the same workload (a bounded number of repetitions, on all host
threads and on one).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "W4A16 GEMM: weight GB/s at M=1 and TFLOP/s at M=4096 vs MI355X roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
REPEATS = 5                  # the timed steps are split into this many repeats

# name -> (format, M, N, K, output dtype name)
WORKLOADS = {
    "tiny_int4_m16": (0, 16, 256, 512, "f32"),
    "decode_gemv_int4_m1": (0, 1, 8192, 3072, "bf16"),
    "nvfp4_m16": (1, 16, 3072, 8192, "bf16"),
    "mxfp4_m4096": (2, 4096, 8192, 3072, "bf16"),
}
CHAIN = "decode_chain_3b_int4_m1"
# int4 g128, NVFP4, MXFP4, int4 g32, int4 g64, symmetric int4 (g128, no zeros)
GROUP = {0: 128, 1: 16, 2: 32, 3: 32, 4: 64, 5: 128}
INT4_FORMATS = (0, 3, 4, 5)  # bf16 scales
ZERO_FORMATS = (0, 3, 4)     # with a zero array


def algorithmic_bytes(fmt, M, N, K, out):
    """Bytes the method must move once: packed + scales (+ zeros) + A + C."""
    G = GROUP[fmt]
    int4 = fmt in INT4_FORMATS
    ng = (K + G - 1) // G  # groups per row (the last may be shorter)
    weight = N * K // 2 + N * ng * (2 if int4 else 1) + (N * ng if fmt in ZERO_FORMATS else 0)
    io = M * K * 2 + M * N * (4 if out == "f32" else 2)
    return weight, weight + io


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


CSRC = "weight_only_bit_w4a16_amd/csrc/"
KERNEL_SOURCES = {
    "skinny": [CSRC + "skinny.hip", CSRC + "common.hpp"],
    "mid": [CSRC + "mid.hip", CSRC + "common.hpp"],
    "tiled": [CSRC + "tiled.hip", CSRC + "common.hpp"],
}


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch (per pass for the decode chain) from the committed
    rocprofv3 counter summary profiles/traffic_<kernel>_<workload>.txt (lines
    "key value"), or None when there is none or the kernel's source changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and not line.startswith("#"):
                rec[parts[0]] = parts[1]
    if rec.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    # per launch, or per pass for the decode chain (one batched call)
    return int(float(rec.get("hbm_bytes_per_launch", rec.get("hbm_bytes_per_step"))))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def hbm_roofline(bytes_per_launch, launch_ms, kernel, workload, traffic=True):
    ach = bytes_per_launch / (launch_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile(kernel, workload) if traffic else None,
            "kernel": kernel, "mean_launch_us": round(launch_ms * 1e3, 3),
            "bytes_per_launch": int(bytes_per_launch)}


def mfma_roofline(flops, launch_ms, kernel, workload, traffic=True):
    ach = flops / (launch_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_from_profile(kernel, workload) if traffic else None,
            "kernel": kernel, "mean_launch_us": round(launch_ms * 1e3, 3), "flops_per_launch": flops}


def batched_launches(shapes, per_launch=32):
    """Launches of one w4a16_gemm_batched call at M <= 16: one per (K, N) and
    32 items (the library's grouping)."""
    count = {}
    for _, n, k in shapes:
        count[(k, n)] = count.get((k, n), 0) + 1
    return sum(-(-c // per_launch) for c in count.values())


def progress(msg):
    """One line on stderr per finished piece of work (the JSON line is stdout)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode_gemv_int4_m1", choices=list(WORKLOADS) + [CHAIN])
    ap.add_argument("--path", default="auto", choices=["auto", "skinny", "mid", "tiled"])
    ap.add_argument("--shape", default=None,
                    help="custom single-GEMM workload 'format,M,N,K' (format 0 int4 g128, 1 nvfp4, "
                         "2 mxfp4, 3 int4 g32, 4 int4 g64, 5 symmetric int4; bf16 out) instead of --workload")
    ap.add_argument("--epilogue", default=None, choices=["none", "relu", "silu", "gelu_tanh"],
                    help="single-GEMM workloads: fuse a bf16 bias, a residual (beta = 1) and this "
                         "activation into the GEMM (w4a16_gemm_ex); their bytes count as traffic")
    ap.add_argument("--prepacked", action="store_true",
                    help="time the weights in the library's prepacked layout (w4a16_prepack, untimed; "
                         "K % 128 == 0) instead of the row-major one")
    ap.add_argument("--copies", type=int, default=0,
                    help="distinct weight copies to rotate over (0: enough for >= 1 GiB)")
    ap.add_argument("--side-steps", type=int, default=300,
                    help="timed steps of each additional workload on the default line")
    ap.add_argument("--no-side", action="store_true",
                    help="default line: time the decode GEMV only")
    ap.add_argument("--no-ungrouped", action="store_true",
                    help="decode chain: skip timing the 197 ungrouped launches")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bounds", action="store_true",
                    help="only measure the bounds the kernels are compared with, with the measurement "
                         "kernels of libw4a16_probe.so: the empty-launch floor, a plain read of the decode "
                         "GEMV's weight bytes and of 256 MiB, the MFMA rate of a matrix-only loop, and a "
                         "split-K hand-off between workgroups; one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 10 times (reference "
                         "kernel of known traffic for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.shape:
        f, m, n, k = (int(x) for x in args.shape.split(","))
        name = f"custom_f{f}_m{m}_n{n}_k{k}"
        WORKLOADS[name] = (f, m, n, k, "bf16")
        args.workload = name

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the W4A16 GEMM here runs on a single MI355X "
              "(no multi-GPU path is built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import weight_only_bit_w4a16_amd as w4
    from weight_only_bit_w4a16_amd import inputs

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (torch.cuda.is_available() is False)")
    dev = torch.device("cuda", 0)
    w4.load_library()  # fails loudly if the HIP library is not built

    if args.copy_calibration:
        nbytes = 256 << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_dispatch": nbytes, "dispatches": 10}))
        return

    def to_dev(case):
        A = torch.from_numpy(case.A.view(np.int16)).to(dev).view(torch.bfloat16)
        p = torch.from_numpy(case.packed).to(dev)
        if case.fmt in INT4_FORMATS:
            s = torch.from_numpy(case.scales.view(np.int16)).to(dev).view(torch.bfloat16)
            z = torch.from_numpy(case.zeros).to(dev) if case.zeros is not None else None
        else:
            s = torch.from_numpy(case.scales).to(dev)
            z = None
        return A, p, s, z

    # spin-kernel calibration: cycles per ms of torch.cuda._sleep
    def spin_cycles_per_ms():
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(2_000_000)
        e1.record()
        torch.cuda.synchronize()
        return 2_000_000 / max(e0.elapsed_time(e1), 1e-3)

    cyc_per_ms = spin_cycles_per_ms()

    def measure_bounds():
        """The bounds the kernels are compared with: launch floor, read and MFMA ceilings and the
        split-K hand-off, measured by the kernels of libw4a16_probe.so."""
        import ctypes
        from weight_only_bit_w4a16_amd import _build
        if not os.path.exists(_build.PROBE_LIB):
            raise SystemExit(f"{_build.PROBE_LIB} is missing: build first (__graft_entry__.build())")
        lib = ctypes.CDLL(_build.PROBE_LIB)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.w4a16_probe_empty.argtypes = [P, P]
        lib.w4a16_probe_read.argtypes = [P, I64, I, I, P, P]
        lib.w4a16_probe_mfma.argtypes = [I, I, I, P, P]
        lib.w4a16_probe_handoff.argtypes = [P, P, P, I, I, I, P]
        st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        sink = torch.zeros(16, dtype=torch.int32, device=dev)

        def call(fn, *a):
            def f():
                rc = fn(*a, st())
                if rc != 0:
                    raise RuntimeError(f"probe call failed: {rc}")
            return f

        out = {}
        steps = 1000
        out["empty_launch_us"] = round(timed_graph([[call(lib.w4a16_probe_empty, sink.data_ptr())]], steps, 50)
                                       / steps * 1e3, 3)
        progress(f"bounds: empty launch {out['empty_launch_us']} us per graph node")
        shapes = [(256, 1), (512, 1), (768, 1), (768, 2), (1024, 2), (1024, 4), (512, 8)]
        for name, nbytes in (("decode_gemv_weight_bytes", algorithmic_bytes(0, 1, 8192, 3072, "bf16")[0] // 16 * 16),
                             ("read_256MiB", 256 << 20)):
            copies = max(1, math.ceil((1 << 30) / nbytes)) + 1
            bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
            best = None
            nst = 400 if nbytes < (64 << 20) else 40
            for thr, per in shapes:
                calls = [[call(lib.w4a16_probe_read, b.data_ptr(), nbytes, thr, per, sink.data_ptr())] for b in bufs]
                us = timed_graph(calls, nst, 10) / nst * 1e3
                if best is None or us < best[0]:
                    best = (us, thr, per)
            del bufs
            out[name] = {"bytes": nbytes, "best_us": round(best[0], 3), "threads": best[1], "loads_per_thread": best[2],
                         "tb_per_s": round(nbytes / (best[0] * 1e-6) / 1e12, 3)}
            progress(f"bounds: plain read of {nbytes} B: {best[0]:.3f} us ({out[name]['tb_per_s']} TB/s)")
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        iters = 20000
        f = call(lib.w4a16_probe_mfma, cus, 512, iters, sink.data_ptr())
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        flops = cus * 8 * iters * 8 * 16384.0
        out["mfma_only"] = {"workgroups": cus, "waves_per_workgroup": 8, "ms": round(ms, 3),
                            "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        progress(f"bounds: MFMA-only loop {out['mfma_only']['tflops']} TFLOP/s")
        groups = 64
        hand = {}
        for slices in (2, 4):
            scratch = torch.zeros(groups * slices * 768, dtype=torch.float32, device=dev)
            counters = torch.zeros(groups, dtype=torch.int32, device=dev)
            o = torch.zeros(groups * 768, dtype=torch.float32, device=dev)
            for mode, mname in ((0, "partials_only"), (1, "fence_per_workgroup"), (2, "fence_per_thread"),
                                (3, "second_kernel")):
                c = call(lib.w4a16_probe_handoff, scratch.data_ptr(), counters.data_ptr(), o.data_ptr(),
                         groups, slices, mode)
                hand[f"{slices}_slices_{mname}_us"] = round(timed_graph([[c]], 200, 10) / 200 * 1e3, 3)
            torch.cuda.synchronize()
            if int(counters.abs().sum().item()) != 0:
                raise RuntimeError("hand-off counters not left at zero")
        out["splitk_handoff"] = dict(workgroups_per_slice=groups, **hand)
        progress(f"bounds: split-K hand-off {hand}")
        return {"bounds": out, "device": torch.cuda.get_device_name(dev)}


    def timed(calls_per_step, steps, warmup, graph=False, min_warm_ms=50.0):
        """Time `steps` steps; step i runs the prepared calls
        calls_per_step[i % len(calls_per_step)].  Returns (total ms between
        HIP events around the timed steps, per-step ms of each of the
        REPEATS equal parts).  Warm-up: `warmup` steps, then whole passes over
        every rotation until >= 2 passes and >= min_warm_ms of GPU time.
        Eager: a spin kernel first fills the stream so the launches queue up
        and run back to back.  Graph: each rotation's calls are captured
        once into a HIP graph and the graphs are replayed."""
        nrot = len(calls_per_step)
        runs = [None] * nrot
        if graph:
            for r in range(nrot):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for c in calls_per_step[r]:
                        c()
                runs[r] = g

        def one(i):
            if graph:
                runs[i % nrot].replay()
            else:
                for c in calls_per_step[i % nrot]:
                    c()

        for i in range(warmup):
            one(i)
        torch.cuda.synchronize()
        t0, passes = time.perf_counter(), 0
        while passes < 2 or (time.perf_counter() - t0) * 1e3 < min_warm_ms:
            for i in range(nrot):
                one(i)
            torch.cuda.synchronize()
            passes += 1
        step_ms = (time.perf_counter() - t0) * 1e3 / (passes * nrot)  # upper bound (host-paced)
        # untimed steps queued behind the spin kernel, >= ~1 ms of GPU work,
        # so the timed steps start at working clocks (the spin idles the GPU)
        pre = max(8, min(4000, math.ceil(1.0 / max(step_ms, 1e-4))))
        launches = (steps + pre) * len(calls_per_step[0])
        # each event recorded between launches costs about a launch gap, so a
        # short run keeps the one pair around all of its steps
        parts = REPEATS if steps >= 100 * REPEATS else 1
        bounds = [round(steps * j / parts) for j in range(parts + 1)]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(parts + 1)]
        # queue fill: ~10 us of host time per eager launch (~50 per replay), plus margin
        torch.cuda._sleep(int(cyc_per_ms * (((0.05 * (steps + pre)) if graph else (0.010 * launches)) + 20.0)))
        for i in range(pre):
            one(steps + i)
        ev[0].record()
        for j in range(parts):
            for i in range(bounds[j], bounds[j + 1]):
                one(i)
            ev[j + 1].record()
        torch.cuda.synchronize()
        per = [ev[j].elapsed_time(ev[j + 1]) / (bounds[j + 1] - bounds[j]) for j in range(parts)]
        return ev[0].elapsed_time(ev[parts]), per

    def timed_graph(calls_per_step, steps, warmup):
        """The same steps captured into ONE HIP graph of exactly `steps`
        steps (step i runs calls_per_step[i % len]); after the eager warm-up
        and a replay, the graph is replayed untimed (about 1 ms of work,
        behind the queue-fill spin) and then once between two HIP events.
        Returns the timed replay's ms."""
        nrot = len(calls_per_step)
        for i in range(max(warmup, nrot)):
            for c in calls_per_step[i % nrot]:
                c()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                for c in calls_per_step[i % nrot]:
                    c()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        once_ms = (time.perf_counter() - t0) * 1e3
        pre = max(1, min(200, math.ceil(1.0 / max(once_ms, 1e-3))))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(cyc_per_ms * (0.05 * pre + 5.0)))
        for _ in range(pre):
            g.replay()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    if args.bounds:
        print(json.dumps(measure_bounds()))
        return

    def measure_single(fmt, M, N, K, out, steps, warmup, epilogue=None):
        """One GEMM workload timed over `steps` launches that rotate over
        enough distinct weight copies (>= 1 GiB together) that every launch
        reads its weights from HBM."""
        case = inputs.make_case(fmt, M, N, K, seed=0)
        A, p, s, z = to_dev(case)
        _, tbytes = algorithmic_bytes(fmt, M, N, K, out)
        copies = args.copies or max(1, min(128, math.ceil((1 << 30) / tbytes)))
        odt = torch.float32 if out == "f32" else torch.bfloat16
        C = torch.empty((M, N), dtype=odt, device=dev)
        epi = {}
        if epilogue:
            g = torch.Generator(device="cpu").manual_seed(1)
            epi = dict(bias=torch.randn(N, generator=g).to(dev, torch.bfloat16),
                       residual=torch.randn((M, N), generator=g).to(dev, odt),
                       alpha=1.0, beta=1.0, activation=epilogue)
        calls = []
        for r in range(copies):
            pr = p if r == 0 else p.clone()
            if args.prepacked:
                pr = w4.prepack(pr)
            sr = s if r == 0 else s.clone()
            zr = z if (r == 0 or z is None) else z.clone()
            calls.append([w4.PreparedGemm(fmt, A, pr, sr, zr, C, path=args.path, **epi)])
        eager, per = timed(calls, steps, warmup)
        total = timed_graph(calls, steps, warmup)
        kernel = calls[0][0].kernel
        del calls, C
        vendor_ms = None
        if M > 16 and not epilogue:
            # context for the compute-bound shape: the platform's own dense bf16
            # GEMM (torch.matmul -> hipBLASLt) on the same shape, with the
            # weights already dequantised to bf16 (no 4-bit decode at all)
            W = w4.dequant(fmt, p, s, z)
            Wt = W.t().contiguous()
            Cv = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            vsteps = max(1, min(steps, 200))
            vendor_ms = timed_graph([[lambda: torch.matmul(A, Wt, out=Cv)]], vsteps, warmup) / vsteps
            del W, Wt, Cv
            progress(f"  dense bf16 torch.matmul, same shape: {vendor_ms * 1e3:.3f} us per launch (graph)")
        progress(f"{w4.FORMAT_NAMES[fmt]} M={M} N={N} K={K}: {total / steps * 1e3:.3f} us per launch "
                 f"(graph), {eager / steps * 1e3:.3f} eager ({kernel}, {steps} steps)")
        return {"case": case, "ms": total / steps, "eager_ms": eager / steps,
                "eager_median_ms": statistics.median(per), "copies": copies, "kernel": kernel,
                "vendor_ms": vendor_ms}

    def vendor_entry(r, M, N, K):
        """The dense bf16 GEMM beside a compute-bound workload (context only)."""
        if r.get("vendor_ms") is None:
            return None
        return {"what": "torch.matmul (hipBLASLt) of bf16 A and the dequantised bf16 weights, same "
                        "shape, graph-timed like the workload: the platform's dense GEMM with no "
                        "4-bit decode (context, not the baseline)",
                "ms_per_step": round(r["vendor_ms"], 6),
                "tflops": round(2.0 * M * N * K / (r["vendor_ms"] * 1e-3) / 1e12, 1),
                "w4a16_speedup": round(r["vendor_ms"] / r["ms"], 3)}

    def single_entry(name, steps, warmup):
        fmt, M, N, K, out = WORKLOADS[name]
        r = measure_single(fmt, M, N, K, out, steps, warmup)
        wbytes, tbytes = algorithmic_bytes(fmt, M, N, K, out)
        e = {"workload": name, "format": w4.FORMAT_NAMES[fmt], "M": M, "N": N, "K": K, "out": out,
             "kernel": r["kernel"], "steps": steps, "weight_copies": r["copies"],
             "timing": "hip_graph_replay", "ms_per_step": round(r["ms"], 6),
             "eager_ms_per_step": round(r["eager_ms"], 6),
             "eager_median_ms_per_step": round(r["eager_median_ms"], 6)}
        if M > 16:
            e["tflops"] = round(2.0 * M * N * K / (r["ms"] * 1e-3) / 1e12, 1)
            e["roofline"] = mfma_roofline(2 * M * N * K, r["ms"], r["kernel"], name)
            e["dense_bf16_gemm"] = vendor_entry(r, M, N, K)
        else:
            e["weight_gbs"] = round(wbytes / (r["ms"] * 1e-3) / 1e9, 1)
            e["roofline"] = hbm_roofline(tbytes, r["ms"], r["kernel"], name)
        return e, r

    def measure_chain(steps, warmup, ungrouped=True):
        """The 197 int4 GEMVs of a 3B decoder's decode step (per layer q, k,
        v, o, gate, up, down, then the LM head), each with its own A, timed as
        replays of one captured HIP graph per pass.  The workload's GEMVs are
        independent, so one batched call runs the pass (a launch per shape
        and 32 matrices); a decoder's layer order would allow grouping only
        the matrices of one layer that read the same input, which is timed
        beside it (113 launches), and so are 197 single launches."""
        shapes = inputs.decoder_chain_shapes()
        calls, wbytes, tbytes = [], 0, 0
        out = torch.empty((1, max(n for _, n, _ in shapes)), dtype=torch.bfloat16, device=dev)
        dev_w, dev_a = [], []
        for i, (_, n, k) in enumerate(shapes):
            case = inputs.make_case(0, 1, n, k, inputs.chain_seed(0, i))
            A, p, s, z = to_dev(case)
            if args.prepacked:
                p = w4.prepack(p)
            dev_w.append((p, s, z))
            dev_a.append(A)
            calls.append(w4.PreparedGemm(0, A, p, s, z, out[:, :n], path=args.path))
            wb, tb = algorithmic_bytes(0, 1, n, k, "bf16")
            wbytes += wb
            tbytes += tb
        # matrices that read the same input in one launch
        gcalls = []
        for grp in inputs.decoder_chain_groups():
            A = dev_a[grp[0]]
            if len(grp) == 1:
                gcalls.append(calls[grp[0]])
                continue
            outs = [torch.empty((1, shapes[i][1]), dtype=torch.bfloat16, device=dev) for i in grp]
            gcalls.append(w4.PreparedGroupedGemm(0, A, [dev_w[i] for i in grp], outs, path=args.path))
        bouts = [torch.empty((1, n), dtype=torch.bfloat16, device=dev) for _, n, _ in shapes]
        bcall = w4.PreparedBatchedGemm(0, [(dev_a[i], *dev_w[i]) for i in range(len(shapes))], bouts)
        blaunches = batched_launches(shapes)
        esteps = max(1, steps // 10)
        eager_ms = timed([[bcall]], esteps, warmup)[0] / esteps
        lsteps = max(1, min(steps, 50))  # graphs of 113 / 197 launches per step
        layer_ms = timed_graph([gcalls], lsteps, warmup) / lsteps
        ungrouped_ms = timed_graph([calls], lsteps, warmup) / lsteps if ungrouped else None
        total_ms = timed_graph([[bcall]], steps, warmup)
        ms = total_ms / steps
        per = [ms]
        progress(f"decode chain: {ms * 1e3:.1f} us per pass (batched, graph), eager {eager_ms * 1e3:.1f} us, "
                 f"layer-grouped {layer_ms * 1e3:.1f} us")
        e = {"workload": CHAIN, "matrices": len(calls), "M": 1, "format": "int4_g128", "out": "bf16",
             "call": "w4a16_gemm_batched", "launches_per_step": blaunches,
             "weights": "prepacked" if args.prepacked else "row-major",
             "grouping": "independent GEMVs: one launch per (K, N) and 32 matrices",
             "timing": "hip_graph_replay", "steps": steps, "ms_per_step": round(ms, 6),
             "eager_ms_per_step": round(eager_ms, 4),
             "layer_grouped_launches_per_step": len(gcalls),
             "layer_grouping": "per layer [q,k,v] [o] [gate,up] [down], then [lm_head] (w4a16_gemm_grouped)",
             "layer_grouped_ms_per_step": round(layer_ms, 4),
             "ungrouped_launches_per_step": len(calls),
             "ungrouped_ms_per_step": None if ungrouped_ms is None else round(ungrouped_ms, 4),
             "weight_gbs": round(wbytes / (ms * 1e-3) / 1e9, 1)}
        # the roofline of the whole pass: all its bytes over the step time
        e["roofline"] = hbm_roofline(tbytes, ms, calls[0].kernel, CHAIN)
        e["roofline"]["bytes_per_launch"] = None
        e["roofline"]["bytes_per_step"] = int(tbytes)
        e["roofline"]["mean_launch_us"] = round(ms * 1e3 / blaunches, 3)
        return e, wbytes

    if args.workload == CHAIN:
        e, wbytes = measure_chain(args.steps, args.warmup, ungrouped=not args.no_ungrouped)
        ms = e["ms_per_step"]
        value, unit = wbytes / (ms * 1e-3) / 1e9, "GB/s"
        roof = e.pop("roofline")
        config = e
    else:
        fmt, M, N, K, out = WORKLOADS[args.workload]
        r = measure_single(fmt, M, N, K, out, args.steps, args.warmup, epilogue=args.epilogue)
        ms = r["ms"]
        wbytes, tbytes = algorithmic_bytes(fmt, M, N, K, out)
        if args.epilogue:  # + bias (bf16) + residual (C's dtype)
            tbytes += N * 2 + M * N * (4 if out == "f32" else 2)
        config = {"workload": args.workload, "format": w4.FORMAT_NAMES[fmt], "M": M, "N": N, "K": K,
                  "weights": "prepacked" if args.prepacked else "row-major",
                  "out": out, "weight_copies": r["copies"], "kernel": r["kernel"],
                  "timing": "hip_graph_replay", "eager_ms_per_step": round(r["eager_ms"], 6),
                  "eager_median_ms_per_step": round(r["eager_median_ms"], 6)}
        if args.epilogue:
            config["epilogue"] = {"bias": "bf16", "residual": out, "beta": 1.0,
                                  "activation": args.epilogue}
        if M > 16:
            value, unit = 2.0 * M * N * K / (ms * 1e-3) / 1e12, "TFLOP/s"
            roof = mfma_roofline(2 * M * N * K, ms, r["kernel"], args.workload, traffic=not args.epilogue)
            config["dense_bf16_gemm"] = vendor_entry(r, M, N, K)
        else:
            value, unit = wbytes / (ms * 1e-3) / 1e9, "GB/s"
            roof = hbm_roofline(tbytes, ms, r["kernel"], args.workload, traffic=not args.epilogue)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "roofline": roof,
    }

    # ---- the metric's other workloads, each with its own roofline -------------
    if args.workload == "decode_gemv_int4_m1" and not args.no_side and not args.shape:
        side = {}
        for name in ("tiny_int4_m16", "nvfp4_m16", "mxfp4_m4096"):
            side[name] = single_entry(name, args.side_steps, 10)[0]
        side[CHAIN] = measure_chain(min(args.side_steps, 200), 5)[0]
        result["workloads"] = side

    # ---- CPU baseline: the oracle on the same workload ------------------------
    if not args.no_cpu_baseline and args.workload != CHAIN and not args.shape:
        import oracle
        fmt, M, N, K, out = WORKLOADS[args.workload]
        case = inputs.make_case(fmt, M, N, K, seed=0)
        if M > 16:
            # 256 sampled outputs per repetition (the full product is 103 G MACs)
            rng = np.random.default_rng(0)
            mi, ni = rng.integers(0, M, 256), rng.integers(0, N, 256)
            fn = lambda: oracle.gemm_at(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K, mi, ni)
            per_rep_units = 2.0 * 256 * K / 1e12
            cunit, sample = "TFLOP/s", f"256 sampled outputs of the {args.workload} GEMM per repetition"
        else:
            fn = lambda: oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
            per_rep_units = wbytes / 1e9
            cunit = "GB/s"
            sample = f"the full {args.workload} GEMM (M={M}, N={N}, K={K}) per repetition"

        def rate(seconds):
            fn()  # warm
            reps, t0 = 0, time.perf_counter()
            while True:
                fn()
                reps += 1
                el = time.perf_counter() - t0
                if el >= seconds:
                    return per_rep_units * reps / el, reps, el

        threads = oracle.num_threads()
        v_all, reps, el = rate(args.cpu_seconds)
        progress(f"cpu baseline: {v_all:.4f} {cunit} on {threads} threads")
        oracle.set_num_threads(1)
        v_one, reps1, el1 = rate(max(1.0, args.cpu_seconds / 2))
        # the dequantisation alone (single-threaded loop in the oracle)
        t0 = time.perf_counter()
        oracle.dequant(fmt, case.packed, case.scales, case.zeros, N, K)
        dq_s = time.perf_counter() - t0
        oracle.set_num_threads(threads)
        result["cpu_baseline"] = {
            "value": round(v_all, 6), "unit": cunit, "cores": threads, "kind": "oracle",
            "sample": f"{sample}, {reps} repetitions in {el:.1f} s on {threads} threads "
                      "(plain fp64 C oracle, OpenMP over output rows)",
            "single_thread_value": round(v_one, 6),
            "single_thread_sample": f"{reps1} repetitions in {el1:.1f} s on 1 thread",
            "dequant_ms": round(dq_s * 1e3, 1),
            "dequant_sample": f"oracle dequantisation of the {N} x {K} weights, once, 1 thread",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
