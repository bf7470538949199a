"""Benchmark of D = A.B + C on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one D = A.B + C call on the workload, inputs already resident in
HBM.  W untimed steps, then exactly K timed steps bracketed by device
synchronisation; the GEMM kernel's average duration is taken with HIP events
recorded on the stream the kernel is launched on (torch's current stream).
Prints one JSON line.  The default workload is the 4096^3 bf16 GEMM with fp32
C and D; the same run then times the 8192^3 block-scaled fp8 GEMM (e4m3 with
e8m0 scales per 32 K, fp32 D) the same way and reports it under
"secondary", with its own roofline and CPU baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s and % of MI355X MFMA peak (bf16 4096³; mxfp8 8192³)"
# MI355X published dense peaks (256 CUs at 2.4 GHz), TFLOP/s
PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "e4m3": 5033.2, "e2m3": 10066.3, "e3m2": 10066.3,
               "e2m1": 10066.3}
# bytes per element of A and B
ELEMENT_BYTES = {"e4m3": 1.0, "e2m3": 0.75, "e3m2": 0.75, "e2m1": 0.5}


def algorithmic_bytes(w):
    """Bytes the operation must move at least once: A, B, (C), D, (scales)."""
    es = ELEMENT_BYTES.get(w.in_type, 2.0)
    os_ = 4 if w.out_type == "f32" else 2
    b = int((w.M * w.K + w.N * w.K) * es) + w.M * w.N * os_
    if w.dist_c is not None:
        b += w.M * w.N * os_
    if w.scaled:
        b += (w.M + w.N) * (w.K // 32)
    return b


def measured_traffic(w):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when there is none or the kernels changed since."""
    from rocprof_summary import PROFILES, kernel_source_hash
    path = os.path.join(PROFILES, "%s_traffic.json" % w.name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    if doc.get("kernel_sources") != kernel_source_hash(w.name):
        return None
    return int(round(doc["traffic_bytes_per_launch"]))


def device_inputs(w, x, torch):
    dev = torch.device("cuda:0")
    if w.in_type in ELEMENT_BYTES:
        A = torch.from_numpy(x["A"]).to(dev)
        B = torch.from_numpy(x["B"]).to(dev)
        extra = (torch.from_numpy(x["SFA"]).to(dev), torch.from_numpy(x["SFB"]).to(dev))
    else:
        import numpy as np
        dt = torch.bfloat16 if w.in_type == "bf16" else torch.float16
        A = torch.from_numpy(x["A"].view(np.int16)).view(dt).to(dev)
        B = torch.from_numpy(x["B"].view(np.int16)).view(dt).to(dev)
        extra = None
    C = torch.from_numpy(x["C"]).to(dev) if x["C"] is not None else None
    return A, B, C, extra


def cpu_model():
    """The host CPU's model name (first processor of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, target_rows):
    """Time the oracle on the first `target_rows` full rows of D (every column),
    on every host thread OpenMP gives it."""
    import numpy as np
    import oracle
    rows = min(target_rows, w.M)
    idx = np.arange(rows * w.N, dtype=np.int64)
    cores = oracle.num_threads()
    s1 = (lambda s: s[:1] if s is not None else None)
    oracle.gemm_ref(w.in_type, x["A"][:1], x["B"][:1], C=None, SFA=s1(x["SFA"]), SFB=s1(x["SFB"]),
                    idx=np.zeros(1, np.int64), nthreads=cores)  # load, warm
    t0 = time.perf_counter()
    oracle.gemm_ref(w.in_type, x["A"], x["B"], C=x["C"], SFA=x["SFA"], SFB=x["SFB"], idx=idx, nthreads=cores)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "first %d rows x all %d columns of D (%d elements, each a full K=%d fp64 dot product); "
                      "%.1f s" % (rows, w.N, rows * w.N, w.K, dt)}


def cpu_small_full():
    """The oracle on the whole 256^3 bf16 workload (every element), on all
    host threads and on one thread: the median of three runs each."""
    import oracle
    from tiled_dense_gemm_tile_amd import inputs
    w = inputs.WORKLOADS["square256_bf16"]
    x = inputs.generate(w)
    cores = oracle.num_threads()
    out = {"workload": w.name, "elements": w.M * w.N, "cpu_model": cpu_model()}
    for key, nt in (("all_threads", cores), ("one_thread", 1)):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.gemm_ref("bf16", x["A"], x["B"], C=x["C"], nthreads=nt)
            ts.append(time.perf_counter() - t0)
        t = sorted(ts)[1]
        out[key] = {"threads": nt, "seconds": round(t, 5), "TFLOP/s": w.flops / t / 1e12}
    oracle.gemm_ref("bf16", x["A"][:1], x["B"][:1], nthreads=cores)    # leave the thread count as found
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="square4096_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="with the default workload, skip the 8192^3 block-scaled fp8 line (secondary)")
    ap.add_argument("--settle", type=float, default=0.3, metavar="SECONDS",
                    help="untimed run of the same step before the warmup steps, so the timed steps "
                         "see the clocks the GPU holds under sustained load (0 disables)")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of D the CPU baseline evaluates (default: about 1.3e10 multiply-adds)")
    ap.add_argument("--splits", type=int, default=None,
                    help="run the split-K entry point with this many K ranges (0: the library's choice; the "
                         "default for workloads with fewer than 128 output tiles)")
    ap.add_argument("--a-order", choices=("k", "mn"), default="k",
                    help="16-bit workloads: store A K-contiguous (M x K) or MN-contiguous (K x M), same values")
    ap.add_argument("--b-order", choices=("k", "mn"), default="k",
                    help="16-bit workloads: store B K-contiguous (N x K) or MN-contiguous (K x N), same values")
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MiB buffer before every timed step, so no operand is left in L2 or the "
                         "256 MB Infinity Cache; each step is timed alone (events around the GEMM only) and "
                         "value comes from those times, the writes excluded")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 3}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    from tiled_dense_gemm_tile_amd import inputs

    primary = measure(inputs.WORKLOADS[args.workload], args, args.a_order, args.b_order, args.splits)
    res = {"metric": METRIC}
    res.update(primary)
    if args.workload == "square4096_bf16" and not args.no_secondary:
        # the metric's second configuration, timed in the same process the same way
        torch.cuda.empty_cache()
        sec = measure(inputs.WORKLOADS["mxfp8_8192"], args, "k", "k", None)
        res["secondary"] = {k: sec[k] for k in ("value", "unit", "ms_per_step", "dtype", "config", "roofline")
                            if k in sec}
        if "cpu_baseline" in sec:
            res["secondary"]["cpu_baseline"] = sec["cpu_baseline"]
    if not args.no_cpu_baseline:
        res["cpu_baseline"]["small_full"] = cpu_small_full()
    print(json.dumps(res), flush=True)


def measure(w, args, a_order, b_order, splits):
    """Time one workload's step (settle, warmup, then exactly args.steps
    timed steps) and return the JSON fields that describe it."""
    import torch
    import tiled_dense_gemm_tile_amd as tg
    from tiled_dense_gemm_tile_amd import inputs
    x = inputs.generate(w)
    A, B, C, extra = device_inputs(w, x, torch)
    if w.in_type in ("bf16", "fp16"):
        # MN-contiguous storage: the transposed copy, viewed back as (rows, K)
        if a_order == "mn":
            A = A.t().contiguous().t()
        if b_order == "mn":
            B = B.t().contiguous().t()
    out_dtype = torch.float32 if w.out_type == "f32" else torch.bfloat16
    D = torch.empty((w.M, w.N), dtype=out_dtype, device="cuda:0")

    if splits is None and ((w.M + 255) // 256) * ((w.N + 255) // 256) < 128:
        splits = 0
    kernels_per_step = 1
    if w.in_type in ("bf16", "fp16") and splits is not None:
        # split-K: the workspace is allocated once, outside the timed steps
        fn = tg.gemm_bf16_splitk if w.in_type == "bf16" else tg.gemm_fp16_splitk
        nbytes = tg.splitk_workspace_bytes(w.M, w.N, w.K, splits)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda:0") if nbytes else None
        kernels_per_step = 2 if nbytes else 1
        step = lambda: fn(A, B, C, out_dtype=out_dtype, D=D, splits=splits, workspace=ws)
    elif w.in_type == "bf16":
        step = lambda: tg.gemm_bf16(A, B, C, out_dtype=out_dtype, D=D)
    elif w.in_type == "fp16":
        step = lambda: tg.gemm_fp16(A, B, C, out_dtype=out_dtype, D=D)
    else:
        SFA, SFB = extra
        kw = {} if w.in_type not in ("e2m3", "e3m2") else {"fmt": w.in_type}
        if splits is not None:
            # split-K: the workspace is allocated once, outside the timed steps
            nbytes = tg.splitk_workspace_bytes(w.M, w.N, w.K, splits)
            ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda:0") if nbytes else None
            kernels_per_step = 2 if nbytes else 1
            fn = {"e4m3": tg.gemm_mxfp8_splitk, "e2m1": tg.gemm_mxfp4_splitk}.get(w.in_type, tg.gemm_mxfp6_splitk)
            kw.update(splits=splits, workspace=ws)
        else:
            fn = {"e4m3": tg.gemm_mxfp8, "e2m1": tg.gemm_mxfp4}.get(w.in_type, tg.gemm_mxfp6)
        step = lambda: fn(A, SFA, B, SFB, C, out_dtype=out_dtype, D=D, **kw)
        if w.packed:
            # tile images made once, before any timed step
            AP, BP = tg.mxfp6_pack(A), tg.mxfp6_pack(B)
            step = lambda: tg.gemm_mxfp6_packed(AP, SFA, BP, SFB, w.M, w.N, w.K, C, out_dtype=out_dtype, D=D,
                                                **kw)

    # The GPU raises its clocks over the first milliseconds of sustained
    # work; a few warmup launches of a ~0.1 ms kernel end before that, so
    # the same step first runs untimed for about --settle seconds.
    t_settle = time.perf_counter() + args.settle
    while time.perf_counter() < t_settle:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if args.cold:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        for i in range(args.steps):
            flush.fill_(i & 255)
            starts[i].record(stream)
            step()
            ends[i].record(stream)
        torch.cuda.synchronize()
        times = [starts[i].elapsed_time(ends[i]) for i in range(args.steps)]
        per_step = sorted(times)
        kernel_ms = sum(times) / args.steps
        ms_per_step = kernel_ms                        # the flushes are not part of the step
    else:
        # an event before every step and after the last, all on the launch stream
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        t0 = time.perf_counter()
        evs[0].record(stream)
        for i in range(args.steps):
            step()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev0, ev1 = evs[0], evs[-1]
        per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
        # one GEMM launch per step (split-K: the GEMM and the reduction of its partials)
        kernel_ms = ev0.elapsed_time(ev1) / args.steps
        ms_per_step = wall * 1e3 / args.steps

    tflops = w.flops / (kernel_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.in_type]
    res = {
        "value": round(w.flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_type,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "in": w.in_type, "out": w.out_type,
                   "C": "fp32 U[-1,1]" if w.dist_c else "none", "layout": "A row-major, B column-major (N x K)",
                   "seed": w.seed, "note": w.note,
                   "splits": None if splits is None else (splits or "auto"),
                   "caches": "cold (512 MiB written before each step)" if args.cold else "warm",
                   "storage": {"A": "K x M" if a_order == "mn" else "M x K",
                               "B": "K x N" if b_order == "mn" else "N x K"}
                   if not w.packed else "tile images of A and B (gemm_mxfp6_pack), made before the timed steps"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": measured_traffic(w),
                     "kernel_ms": round(kernel_ms, 5), "kernel_ms_median": round(per_step[len(per_step) // 2], 5),
                     "kernel_ms_min": round(per_step[0], 5), "kernels_per_step": kernels_per_step,
                     "algorithmic_bytes": algorithmic_bytes(w)},
    }
    del A, B, C, D, extra, step
    if not args.no_cpu_baseline:
        rows = args.cpu_rows or max(1, int(1.3e10 // (w.N * w.K)))
        res["cpu_baseline"] = cpu_baseline(w, x, rows)
    return res


if __name__ == "__main__":
    main()
