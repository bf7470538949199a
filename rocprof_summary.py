"""Profile the benchmark with rocprofv3 and write short text summaries to profiles/.

    python rocprof_summary.py [--workload square4096_bf16] [--out-dir rocprof_out]
                              [--skip-trace] [--skip-traffic] [--skip-counters]

Runs, each as its own child process with the program directly after ``--``:

1. ``rocprofv3 --kernel-trace --stats`` of ``bench.py`` (the benchmark's
   own command line, no CPU baseline) -> ``profiles/<kernel>_<workload>_trace.txt``
   with the per-kernel average duration;
2. two ``--pmc`` passes (FETCH_SIZE, then WRITE_SIZE) over the same command
   and over ``bench.py --calibrate-copy 256`` (a plain device copy of known
   size), giving the HBM bytes per GEMM launch after scaling each counter by
   the copy's bytes / reading -> ``profiles/<workload>_traffic.json`` (read by
   bench.py while the kernel sources still hash to the recorded value);
3. counter passes for MFMA activity and LDS bank conflicts ->
   ``profiles/<workload>_counters.txt``.

This process itself never touches the GPU.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import shlex
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "tiled_dense_gemm_tile_amd", "csrc")
COPY_MIB = 256


def instance_file(in_type: str, out_type: str) -> str:
    """The translation unit holding a workload's kernels."""
    if in_type in ("bf16", "fp16"):
        return "f16_%s_%s.hip" % (in_type, out_type)
    return "%s_%s.hip" % ({"e4m3": "mx", "e2m3": "mx6", "e3m2": "mx6", "e2m1": "mx4"}[in_type], out_type)


def _include_closure(name, seen):
    if name in seen:
        return
    seen.add(name)
    with open(os.path.join(CSRC, name)) as f:
        for line in f:
            line = line.strip()
            if line.startswith('#include "'):
                inc = line.split('"')[1]
                # (the public header holds declarations only: not hashed)
                if not inc.startswith("..") and os.path.exists(os.path.join(CSRC, inc)):
                    _include_closure(inc, seen)


def kernel_source_hash(workload: str) -> str:
    """Hash of the sources a workload's kernels are built from: its instance
    file and its family's entry-point file (validation and dispatch) with
    everything they include."""
    from tiled_dense_gemm_tile_amd import inputs
    w = inputs.WORKLOADS[workload]
    files = set()
    _include_closure(instance_file(w.in_type, w.out_type), files)
    api = {"e4m3": "mx_api.hip", "e2m3": "mx6_api.hip", "e3m2": "mx6_api.hip",
           "e2m1": "mx4_api.hip"}.get(w.in_type, "tilegemm.hip")
    _include_closure(api, files)
    _include_closure("splitk.hip", files)              # the split-K reduction
    h = hashlib.sha256()
    for f in sorted(files):
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def run(cmd, log):
    print("+", " ".join(shlex.quote(c) for c in cmd), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(cmd, stdout=f, stderr=subprocess.STDOUT, cwd=ROOT)
    if r.returncode != 0:
        with open(log) as f:
            tail = f.read()[-2000:]
        raise SystemExit("command failed (%d):\n%s" % (r.returncode, tail))


def csv_rows(d, pattern):
    files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not files:
        raise SystemExit("no %s under %s" % (pattern, d))
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def counter_per_dispatch(d, name_filter):
    """{dispatch_id: {counter: value}} summed over instances, for kernels whose name matches,
    with the dispatch's duration in ns under "duration_ns"."""
    out = {}
    for r in csv_rows(d, "*counter_collection.csv"):
        if name_filter not in r["Kernel_Name"]:
            continue
        did = int(r["Dispatch_Id"])
        e = out.setdefault(did, {"kernel": r["Kernel_Name"]})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            e["duration_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return out


def pmc(counters, prog, out_dir, tag):
    d = os.path.join(out_dir, tag)
    cmd = ["timeout", "-s", "KILL", "90", "rocprofv3", "--pmc"] + counters + \
          ["--output-format", "csv", "-d", d, "-o", "run", "--"] + prog
    run(cmd, d + ".log")
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="square4096_bf16")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "rocprof_out"))
    ap.add_argument("--skip-trace", action="store_true")
    ap.add_argument("--skip-traffic", action="store_true")
    ap.add_argument("--skip-counters", action="store_true")
    ap.add_argument("--dest", default=PROFILES, help="directory the summaries are written to")
    ap.add_argument("--reparse", action="store_true",
                    help="counters: rewrite the summary from the csv files already under --out-dir "
                         "(no GPU run)")
    args = ap.parse_args()
    os.makedirs(args.out_dir, exist_ok=True)
    os.makedirs(args.dest, exist_ok=True)
    os.environ.setdefault("TMPDIR", "/tmp")
    bench = ["python3", "bench.py", "--workload", args.workload, "--steps", str(args.steps),
             "--warmup", str(args.warmup), "--no-cpu-baseline"]
    short = ["python3", "bench.py", "--workload", args.workload, "--steps", "3", "--warmup", "1",
             "--no-cpu-baseline"]
    kname = "gemm_mx" if "mxfp" in args.workload else "gemm_f16"
    src_hash = kernel_source_hash(args.workload)

    if not args.skip_trace:
        d = os.path.join(args.out_dir, "trace")
        cmd = ["timeout", "-s", "KILL", "300", "rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv",
               "-d", d, "-o", "run", "--"] + bench
        run(cmd, d + ".log")
        stats = csv_rows(d, "*kernel_stats.csv")
        with open(d + ".log") as f:
            bench_line = [l for l in f.read().splitlines() if l.startswith("{")][-1]
        shown = " ".join(cmd[4:]).replace(ROOT + os.sep, "")
        lines = ["# rocprofv3 kernel trace: %s" % args.workload,
                 "command: " + shown, "kernel sources: %s" % src_hash, "",
                 "%-90s %8s %14s %14s" % ("kernel", "calls", "average_ns", "total_ns")]
        main_kernel = None
        for r in stats:
            lines.append("%-90s %8s %14s %14s" % (r["Name"][:90], r["Calls"], r["AverageNs"], r["TotalDurationNs"]))
            if kname in r["Name"] and main_kernel is None:
                main_kernel = r
        b = json.loads(bench_line)
        lines += ["", "bench.py line from the same run:", bench_line]
        if main_kernel:
            lines.append("average %s duration: %.2f us (bench.py HIP-event kernel_ms: %.2f us)"
                         % (kname, float(main_kernel["AverageNs"]) / 1e3, b["roofline"]["kernel_ms"] * 1e3))
        out = os.path.join(args.dest, "%s_%s_trace.txt" % (kname, args.workload))
        with open(out, "w") as f:
            f.write("\n".join(lines) + "\n")
        print("wrote", out)

    if not args.skip_traffic:
        copy = ["python3", "bench.py", "--calibrate-copy", str(COPY_MIB)]
        res = {}
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            dg = pmc([ctr], short, args.out_dir, "pmc_" + ctr.lower())
            dc = pmc([ctr], copy, args.out_dir, "pmc_copy_" + ctr.lower())
            g = [v[ctr] for v in counter_per_dispatch(dg, kname).values()]
            c = [v[ctr] for v in counter_per_dispatch(dc, "copyBuffer").values()]
            if not c:
                c = [v[ctr] for v in counter_per_dispatch(dc, "").values() if v[ctr] > 1024]
            kib_gemm = sorted(g)[len(g) // 2]
            kib_copy = sorted(c)[len(c) // 2]
            factor = COPY_MIB * 1024.0 / kib_copy      # true KiB per counted KiB
            res[ctr] = {"gemm_kib_per_launch": kib_gemm, "copy_kib": kib_copy, "copy_true_kib": COPY_MIB * 1024,
                        "factor": factor, "bytes_per_launch": kib_gemm * 1024.0 * factor}
        total = res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]
        doc = {"workload": args.workload, "kernel_sources": src_hash, "command": " ".join(short),
               "copy_command": " ".join(copy), "counters": res, "traffic_bytes_per_launch": total}
        out = os.path.join(args.dest, "%s_traffic.json" % args.workload)
        with open(out, "w") as f:
            json.dump(doc, f, indent=1)
            f.write("\n")
        print("wrote", out, "traffic %.1f MB per launch" % (total / 1e6))

    if not args.skip_counters:
        # (no MOPS counter is used for fp4 and fp6)
        mops = {"mxfp8": ["SQ_INSTS_VALU_MFMA_MOPS_F8"], "mxfp4": [], "mxfp6": []}.get(args.workload[:5],
                                                                         ["SQ_INSTS_VALU_MFMA_MOPS_BF16"])
        passes = [["GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES"] + mops +
                  ["SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY"],
                  ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS",
                   "SQ_LDS_ADDR_CONFLICT", "SQ_LDS_UNALIGNED_STALL"],
                  ["TCC_HIT", "TCC_MISS"]]
        lines = ["# rocprofv3 counters: %s" % args.workload, "kernel sources: %s" % src_hash, ""]
        for i, pc in enumerate(passes):
            d = os.path.join(args.out_dir, "pmc_pass%d" % i) if args.reparse else pmc(pc, short, args.out_dir,
                                                                                     "pmc_pass%d" % i)
            per = counter_per_dispatch(d, kname)
            did = sorted(per)[-1]
            lines.append("command: rocprofv3 --pmc %s -- %s" % (" ".join(pc), " ".join(short)))
            for c in pc:
                lines.append("  %-30s %18.0f" % (c, per[did].get(c, float("nan"))))
            if "SQ_LDS_BANK_CONFLICT" in pc and per[did].get("SQ_LDS_IDX_ACTIVE"):
                lines.append("  bank-conflict cycles / LDS active cycles = %.4f"
                             % (per[did]["SQ_LDS_BANK_CONFLICT"] / per[did]["SQ_LDS_IDX_ACTIVE"]))
            if "TCC_HIT" in pc:
                h, m = per[did]["TCC_HIT"], per[did]["TCC_MISS"]
                lines.append("  L2 hit rate = %.3f" % (h / (h + m)))
            if "SQ_VALU_MFMA_BUSY_CYCLES" in pc:
                # busy cycles are summed over the 1024 SIMDs, GUI-active cycles over the 8 XCDs
                lines.append("  MFMA busy fraction = (busy / 1024) / (gui_active / 8) = %.3f"
                             % ((per[did]["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024) / (per[did]["GRBM_GUI_ACTIVE"] / 8)))
                if per[did].get("duration_ns"):
                    # (the counters' window can extend past the dispatch's
                    # timestamps, so this overestimates the clock)
                    ghz = per[did]["GRBM_GUI_ACTIVE"] / 8 / per[did]["duration_ns"]
                    lines.append("  clock bound = (gui_active / 8) / dispatch duration = %.3f GHz (%.1f us; an "
                                 "upper bound: gui_active may count past the dispatch's timestamps)"
                                 % (ghz, per[did]["duration_ns"] / 1e3))
            lines.append("")
        out = os.path.join(args.dest, "%s_%s_counters.txt" % (kname, args.workload))
        with open(out, "w") as f:
            f.write("\n".join(lines) + "\n")
        print("wrote", out)


if __name__ == "__main__":
    sys.exit(main())
