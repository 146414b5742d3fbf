#!/usr/bin/env python3
"""Throughput of the W4A16 dequantise-GEMM  C = A . dequant(B)^T  on one MI355X.

Default workload (the M = 1 weight-bandwidth case): decode GEMV with int4
asymmetric group-128 weights, M = 1, N = 8192, K = 3072, bf16 output.  One
step = one w4a16_gemm call.  `value` = weight GB/s = (packed + scales +
zeros bytes) per step / time per step, inputs resident in HBM.  The weights
rotate over enough distinct copies (>= 1 GiB) that no step finds them in the
256 MB last-level cache.  The same line also carries the compute-bound point
of the metric: MXFP4, M = 4096, N = 8192, K = 3072, in TFLOP/s.

Timing: W warm-up steps, then a spin kernel fills the stream so that the K
timed launches run back to back; two HIP events on the launch stream bracket
the K steps, `ms_per_step` = their distance / K, and the roofline's `achieved`
uses the same mean duration per launch.  The 197-GEMV decode chain is
captured once as a HIP graph and replayed (its eager time is reported too).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Inputs are synthetic (seeded numpy draws: A ~ N(0, 1) in bf16, uniform codes,
scales / zeros drawn as the workload states).  The CPU baseline is the plain
fp64 oracle on the same workload (a bounded number of repetitions).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "W4A16 GEMM: weight GB/s at M=1 and TFLOP/s at M=4096 vs MI355X roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published

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


KERNEL_SOURCES = {
    "skinny": ["weight_only_bit_w4a16_amd/csrc/skinny.hip", "weight_only_bit_w4a16_amd/csrc/common.hpp"],
    "tiled": ["weight_only_bit_w4a16_amd/csrc/tiled.hip", "weight_only_bit_w4a16_amd/csrc/common.hpp"],
}


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    profiles/traffic_<kernel>_<workload>.txt (lines "key value"), or None when
    there is none or the kernel's source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and not line.startswith("#"):
                rec[parts[0]] = parts[1]
    if rec.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return int(float(rec["hbm_bytes_per_launch"]))


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
    ap.add_argument("--copies", type=int, default=0,
                    help="distinct weight copies to rotate over (0: enough for >= 1 GiB)")
    ap.add_argument("--m4096-steps", type=int, default=300)
    ap.add_argument("--no-m4096", action="store_true")
    ap.add_argument("--no-ungrouped", action="store_true",
                    help="decode chain: skip timing the 197 ungrouped launches")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    def timed(calls_per_step, steps, warmup, graph=False):
        """Time `steps` steps; step i runs the prepared calls
        calls_per_step[i % len(calls_per_step)].  Returns total ms between
        HIP events recorded on the launch stream around the timed steps.
        Eager: a spin kernel first fills the stream so the launches queue up
        and run back to back.  Graph: each rotation's calls are captured
        once into a HIP graph and the graphs are replayed."""
        nrot = len(calls_per_step)
        for i in range(warmup):
            for c in calls_per_step[i % nrot]:
                c()
        torch.cuda.synchronize()
        runs = [None] * nrot
        if graph:
            for r in range(nrot):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for c in calls_per_step[r]:
                        c()
                runs[r] = g
            for r in range(nrot):
                runs[r].replay()
            torch.cuda.synchronize()
        launches = steps * len(calls_per_step[0])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # queue fill: ~10 us of host time per eager launch (~50 per replay), plus margin
        torch.cuda._sleep(int(cyc_per_ms * (((0.05 * steps) if graph else (0.010 * launches)) + 20.0)))
        e0.record()
        for i in range(steps):
            if graph:
                runs[i % nrot].replay()
            else:
                for c in calls_per_step[i % nrot]:
                    c()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def measure_single(fmt, M, N, K, out, steps, warmup):
        """One GEMM workload timed over `steps` launches that rotate over
        enough distinct weight copies (>= 1 GiB together) that every launch
        reads its weights from HBM.  Returns (case, total ms, copies, kernel)."""
        case = inputs.make_case(fmt, M, N, K, seed=0)
        A, p, s, z = to_dev(case)
        _, tbytes = algorithmic_bytes(fmt, M, N, K, out)
        copies = args.copies or max(1, min(128, math.ceil((1 << 30) / tbytes)))
        odt = torch.float32 if out == "f32" else torch.bfloat16
        C = torch.empty((M, N), dtype=odt, device=dev)
        epi = {}
        if args.epilogue:
            g = torch.Generator(device="cpu").manual_seed(1)
            epi = dict(bias=torch.randn(N, generator=g).to(dev, torch.bfloat16),
                       residual=torch.randn((M, N), generator=g).to(dev, odt),
                       alpha=1.0, beta=1.0, activation=args.epilogue)
        calls = []
        for r in range(copies):
            pr = p if r == 0 else p.clone()
            sr = s if r == 0 else s.clone()
            zr = z if (r == 0 or z is None) else z.clone()
            calls.append([w4.PreparedGemm(fmt, A, pr, sr, zr, C, path=args.path, **epi)])
        total = timed(calls, steps, warmup)
        kernel = calls[0][0].kernel
        del calls, C
        return case, total, copies, kernel

    result = {}
    if args.workload == CHAIN:
        shapes = inputs.decoder_chain_shapes()
        calls, wbytes, tbytes = [], 0, 0
        out = torch.empty((1, max(n for _, n, _ in shapes)), dtype=torch.bfloat16, device=dev)
        dev_w, dev_a = [], []
        for i, (name, n, k) in enumerate(shapes):
            case = inputs.make_case(0, 1, n, k, inputs.chain_seed(0, i))
            A, p, s, z = to_dev(case)
            dev_w.append((p, s, z))
            dev_a.append(A)
            calls.append(w4.PreparedGemm(0, A, p, s, z, out[:, :n], path=args.path))
            wb, tb = algorithmic_bytes(0, 1, n, k, "bf16")
            wbytes += wb
            tbytes += tb
        # the framework's decode step: matrices that read the same input in one launch
        gcalls, gouts = [], []
        for grp in inputs.decoder_chain_groups():
            A = dev_a[grp[0]]
            if len(grp) == 1:
                gcalls.append(calls[grp[0]])
                continue
            outs = [torch.empty((1, shapes[i][1]), dtype=torch.bfloat16, device=dev) for i in grp]
            gouts.append(outs)
            gcalls.append(w4.PreparedGroupedGemm(0, A, [dev_w[i] for i in grp], outs, path=args.path))
        eager_ms = timed([gcalls], max(1, args.steps // 10), args.warmup) / max(1, args.steps // 10)
        ungrouped_ms = None if args.no_ungrouped else \
            timed([calls], args.steps, args.warmup, graph=True) / args.steps
        total_ms = timed([gcalls], args.steps, args.warmup, graph=True)
        ms = total_ms / args.steps
        launches_per_step = len(gcalls)
        kernel = calls[0].kernel
        bytes_per_launch = tbytes / len(gcalls)
        config = {"workload": CHAIN, "matrices": len(calls), "M": 1, "format": "int4_g128",
                  "out": "bf16", "launches_per_step": len(gcalls),
                  "grouping": "per layer [q,k,v] [o] [gate,up] [down], then [lm_head]",
                  "timing": "hip_graph_replay", "eager_ms_per_step": round(eager_ms, 4),
                  "ungrouped_launches_per_step": len(calls),
                  "ungrouped_ms_per_step": None if ungrouped_ms is None else round(ungrouped_ms, 4)}
        value = wbytes / (ms * 1e-3) / 1e9
        unit = "GB/s"
        workload = CHAIN
        weight_bytes = wbytes
    else:
        fmt, M, N, K, out = WORKLOADS[args.workload]
        case, total_ms, copies, kernel = measure_single(fmt, M, N, K, out, args.steps, args.warmup)
        wbytes, tbytes = algorithmic_bytes(fmt, M, N, K, out)
        if args.epilogue:  # + bias (bf16) + residual (C's dtype)
            tbytes += N * 2 + M * N * (4 if out == "f32" else 2)
        ms = total_ms / args.steps
        launches_per_step = 1
        bytes_per_launch = tbytes
        config = {"workload": args.workload, "format": w4.FORMAT_NAMES[fmt], "M": M, "N": N, "K": K,
                  "out": out, "weight_copies": copies, "kernel": kernel}
        if args.epilogue:
            config["epilogue"] = {"bias": "bf16", "residual": out, "beta": 1.0,
                                  "activation": args.epilogue}
        workload = args.workload
        weight_bytes = wbytes
        if M > 16:
            value = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            unit = "TFLOP/s"
        else:
            value = wbytes / (ms * 1e-3) / 1e9
            unit = "GB/s"

    mean_launch_ms = ms / launches_per_step
    if args.workload != CHAIN and WORKLOADS[args.workload][1] > 16:
        fmt, M, N, K, out = WORKLOADS[args.workload]
        ach = 2.0 * M * N * K / (mean_launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                "traffic": None if args.epilogue else traffic_from_profile(kernel, workload)}
    else:
        ach = bytes_per_launch / (mean_launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": None if args.epilogue else traffic_from_profile(kernel, workload)}
    roof["kernel"] = kernel
    roof["mean_launch_us"] = round(mean_launch_ms * 1e3, 3)
    roof["bytes_per_launch"] = int(bytes_per_launch) if unit == "GB/s" else None

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

    # ---- the compute-bound point of the metric: MXFP4 at M = 4096 -------------
    if args.workload == "decode_gemv_int4_m1" and not args.no_m4096:
        fmt, M, N, K, out = WORKLOADS["mxfp4_m4096"]
        _, t4, copies4, kernel4 = measure_single(fmt, M, N, K, out, args.m4096_steps, 10)
        tfl = 2.0 * M * N * K / (t4 / args.m4096_steps * 1e-3) / 1e12
        result["m4096"] = {"workload": "mxfp4_m4096", "kernel": kernel4, "steps": args.m4096_steps,
                           "weight_copies": copies4,
                           "ms_per_step": round(t4 / args.m4096_steps, 4),
                           "tflops": round(tfl, 1), "peak": BF16_PEAK_TFLOPS,
                           "frac": round(tfl / BF16_PEAK_TFLOPS, 4)}

    # ---- CPU baseline: the oracle on the same workload ------------------------
    if not args.no_cpu_baseline and args.workload != CHAIN and not args.shape:
        import oracle
        fmt, M, N, K, out = WORKLOADS[args.workload]
        if args.workload == "mxfp4_m4096":
            # 256 sampled outputs per repetition (the full product is 103 G MACs)
            rng = np.random.default_rng(0)
            mi, ni = rng.integers(0, M, 256), rng.integers(0, N, 256)
            fn = lambda: oracle.gemm_at(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K, mi, ni)
            per_rep_units = 2.0 * 256 * K / 1e12
            cunit, sample = "TFLOP/s", "256 sampled outputs of the M=4096 MXFP4 GEMM per repetition"
        else:
            case = inputs.make_case(fmt, M, N, K, seed=0)
            fn = lambda: oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
            per_rep_units = weight_bytes / 1e9
            cunit = "GB/s"
            sample = f"the full {args.workload} GEMM (M={M}, N={N}, K={K}) per repetition"
        fn()  # warm
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        result["cpu_baseline"] = {"value": round(per_rep_units * reps / el, 6), "unit": cunit,
                                  "cores": oracle.num_threads(), "kind": "oracle",
                                  "sample": f"{sample}, {reps} repetitions in {el:.1f} s "
                                            "(plain fp64 C oracle, OpenMP over output rows)"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
