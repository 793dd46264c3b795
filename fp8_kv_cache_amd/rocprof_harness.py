"""rocprofv3 harness for the library's kernels.

Runs ``bench.py --mode profile`` (a few launches of one target: the operator on
a workload, or one of the neighbouring paths named in variants.py; then the
library's streaming-copy probe over 512 MiB) under rocprofv3, one pass per
counter group, each as a child process with its own time limit:

  trace   --kernel-trace --stats           per-kernel average duration
  fetch   --pmc FETCH_SIZE                 HBM bytes read per dispatch (KiB)
  write   --pmc WRITE_SIZE                 HBM bytes written per dispatch (KiB)
  reqs    --pmc TCC_EA0_RDREQ_{32B,64B,128B}_sum TCC_EA0_RDREQ_sum
                                           read requests by size
  waves   --pmc <wave counters>            occupancy
  bench   --kernel-trace --stats           over bench.py's own run of an operator
                                           workload (its ceilings, warmup and
                                           timed steps; no other workload, variant
                                           or CPU baseline), so that the trace's
                                           durations of exactly the timed steps'
                                           launches can be set beside the bench's
                                           event-timed mean

and writes short text summaries (the figures and the exact commands) to the
output directory.  The copy probe's counters against its known byte count
give the scale factor applied to the operator's counters (on gfx950 with this
ROCm, FETCH_SIZE reads about half of the bytes a copy is known to fetch, while
WRITE_SIZE matches).  FETCH_SIZE's expression counts a read request as 128
bytes only through TCC_BUBBLE, and on gfx950 the 128-byte requests land in its
64-byte term: one scale factor is exact for a kernel whose reads are all
128-byte requests (the copy, the operator) but double-counts 32- and 64-byte
ones.  The reqs pass therefore also counts read bytes from the request-size
counters directly (32, 64 and 128 bytes each), with no calibration.

    python -m fp8_kv_cache_amd.rocprof_harness --workload prefill --out prof_out
    python -m fp8_kv_cache_amd.rocprof_harness --workload mxfp8 --out prof_out
    python -m fp8_kv_cache_amd.rocprof_harness --workload prefill --passes bench --out prof_out
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COPY_KERNEL = "stream_copy"
COPY_BYTES = 512 << 20
REQ_COUNTERS = ("TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum",
                "TCC_EA0_RDREQ_sum")


def kernel_sha(family: str = "op") -> str:
    """Hash of the sources that define a kernel family; the counter summaries
    carry it so that a stale summary is never reported as current."""
    sys.path.insert(0, ROOT)
    from fp8_kv_cache_amd.variants import SOURCES
    h = hashlib.sha256()
    for f in SOURCES[family]:
        h.update(open(os.path.join(PKG, "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, flush=True)


def run_pass(name, rocprof_args, workload, launches, out, timeout, bench_args=None):
    """One rocprofv3 run as a child process: over `bench.py --mode profile`
    (a few launches of the target), or over `bench.py <bench_args>` when
    those are given.  Returns the command and the output directory (and, for
    a bench run, its JSON line)."""
    d = os.path.join(out, name)
    os.makedirs(d, exist_ok=True)
    rel = os.path.relpath(d, ROOT)
    program = bench_args if bench_args is not None else [
        "--mode", "profile", "--workload", workload, "--launches", str(launches)]
    cmd = ["rocprofv3"] + rocprof_args + ["--output-format", "csv", "-d", rel, "-o", name, "--",
                                          "python3", "bench.py"] + program
    log("pass %s: %s" % (name, " ".join(cmd)))
    t0 = time.time()
    res = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=timeout)
    with open(os.path.join(d, "stdout.txt"), "w") as f:
        f.write(res.stdout + "\n--- stderr ---\n" + res.stderr)
    log("pass %s: rc=%d in %.1f s" % (name, res.returncode, time.time() - t0))
    # rocprofv3 itself may end with a signal after the program has finished;
    # the program's own last output says whether it did.
    json_line = next((ln for ln in res.stdout.splitlines() if ln.startswith('{"metric"')), None)
    done = "copies of" in res.stderr if bench_args is None else json_line is not None
    if res.returncode != 0 and not done:
        raise RuntimeError("rocprofv3 pass %s failed (rc %d); see %s" % (name, res.returncode, d))
    return cmd, d, json_line


def find_csv(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, d))
    return hits[-1]


def kernel_stats(d):
    rows = list(csv.DictReader(open(find_csv(d, "kernel_stats.csv"))))
    return rows


def dispatch_durations(d, name):
    """Durations (us) of every dispatch of the kernel called exactly `name`,
    in launch order, from the per-dispatch kernel trace."""
    rows = list(csv.DictReader(open(find_csv(d, "kernel_trace.csv"))))
    hits = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows if r["Kernel_Name"] == name)
    return [(e - b) / 1e3 for b, e in hits]


def main_instance(rows, kernel):
    """The stats row of `kernel`'s most-launched template instance."""
    hits = [r for r in rows if kernel in r["Name"]]
    return max(hits, key=lambda r: int(r["Calls"])) if hits else None


def counter_rows(d):
    return list(csv.DictReader(open(find_csv(d, "counter_collection.csv"))))


def per_dispatch(rows, counter):
    """{kernel name: [value per dispatch]} for one counter (values summed over
    the per-dimension rows of a dispatch)."""
    acc = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        key = (r["Kernel_Name"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in acc.items():
        out.setdefault(name, []).append(v)
    return out


def pick(d, want):
    for name, vals in d.items():
        if want in name:
            return name, vals
    return None, []


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--out", default="prof_out")
    ap.add_argument("--launches", type=int, default=5)
    ap.add_argument("--passes", default="trace,fetch,write,reqs,waves")
    ap.add_argument("--wave-counters", default="OccupancyPercent,MeanOccupancyPerCU,SQ_WAVES")
    ap.add_argument("--bench-steps", type=int, default=20)
    ap.add_argument("--bench-warmup", type=int, default=5)
    args = ap.parse_args()
    sys.path.insert(0, ROOT)
    from fp8_kv_cache_amd import variants as V
    from fp8_kv_cache_amd import workloads as W
    t = V.target(args.workload)
    label, op_kernel, prefix = t.label, t.kernel, t.prefix
    out = os.path.abspath(os.path.join(ROOT, args.out))
    os.makedirs(out, exist_ok=True)
    passes = args.passes.split(",")
    summary = {"workload": label, "kernel": op_kernel, "kernel_sha": kernel_sha(t.family)}
    cmds = {}

    if "trace" in passes:
        cmd, d, _ = run_pass("trace", ["--kernel-trace", "--stats"], args.workload, args.launches,
                             out, 300)
        cmds["trace"] = cmd
        rows = kernel_stats(d)
        lines = ["# rocprofv3 kernel trace, kernel %s, workload %s" % (op_kernel, label),
                 "# command (from the repository root): %s" % " ".join(cmd),
                 "# kernel source sha256[:16] = %s" % summary["kernel_sha"], "",
                 "%-70s %6s %14s %14s %14s" % ("kernel", "calls", "avg_us", "min_us", "max_us")]
        for r in rows:
            name = r["Name"][:70]
            lines.append("%-70s %6s %14.2f %14.2f %14.2f" % (
                name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3))
        top = main_instance(rows, op_kernel)
        if top:
            summary["op_avg_us"] = float(top["AverageNs"]) / 1e3
            summary["op_calls"] = int(top["Calls"])
        lines += ["", "# machine-readable:", json.dumps({
            "workload": label, "kernel": op_kernel, "kernel_sha": summary["kernel_sha"],
            "op_avg_us": summary.get("op_avg_us"), "op_calls": summary.get("op_calls")})]
        text = "\n".join(lines) + "\n"
        open(os.path.join(out, "%s_kernel_trace_%s.txt" % (prefix, label)), "w").write(text)
        log(text)

    fetch = write = None
    if "fetch" in passes:
        cmd, d, _ = run_pass("fetch", ["--pmc", "FETCH_SIZE"], args.workload, 3, out, 180)
        cmds["fetch"] = cmd
        fetch = per_dispatch(counter_rows(d), "FETCH_SIZE")
    if "write" in passes:
        cmd, d, _ = run_pass("write", ["--pmc", "WRITE_SIZE"], args.workload, 3, out, 180)
        cmds["write"] = cmd
        write = per_dispatch(counter_rows(d), "WRITE_SIZE")
    reqs = None
    if "reqs" in passes:
        cmd, d, _ = run_pass("reqs", ["--pmc"] + list(REQ_COUNTERS), args.workload, 3, out, 180)
        cmds["reqs"] = cmd
        rows = counter_rows(d)
        reqs = {c: per_dispatch(rows, c) for c in REQ_COUNTERS}

        def by_size(kernel):
            vals = {c: pick(reqs[c], kernel)[1] for c in REQ_COUNTERS}
            if not all(vals.values()):
                return None, None
            per = [32 * a + 64 * b + 128 * c for a, b, c in zip(
                vals["TCC_EA0_RDREQ_32B_sum"], vals["TCC_EA0_RDREQ_64B_sum"], vals["TCC_EA0_RDREQ_128B_sum"])]
            total = [a + b + c for a, b, c in zip(
                vals["TCC_EA0_RDREQ_32B_sum"], vals["TCC_EA0_RDREQ_64B_sum"], vals["TCC_EA0_RDREQ_128B_sum"])]
            i = per.index(min(per))
            return per[i], {"32B": vals["TCC_EA0_RDREQ_32B_sum"][i], "64B": vals["TCC_EA0_RDREQ_64B_sum"][i],
                            "128B": vals["TCC_EA0_RDREQ_128B_sum"][i], "all": vals["TCC_EA0_RDREQ_sum"][i],
                            "sized": total[i]}

        summary["op_read_bytes_by_request"], summary["op_read_requests"] = by_size(op_kernel)
        summary["copy_read_bytes_by_request"], summary["copy_read_requests"] = by_size(COPY_KERNEL)
    if fetch is not None and write is not None:
        op_name, op_f = pick(fetch, op_kernel)
        _, op_w = pick(write, op_kernel)
        cp_name, cp_f = pick(fetch, COPY_KERNEL)
        _, cp_w = pick(write, COPY_KERNEL)
        kib = 1024.0
        # The counters report KiB per dispatch; the copy moves COPY_BYTES each
        # way, which calibrates them.
        f_scale = COPY_BYTES / (min(cp_f) * kib) if cp_f else 1.0
        w_scale = COPY_BYTES / (min(cp_w) * kib) if cp_w else 1.0
        op_fetch = min(op_f) * kib if op_f else None
        op_write = min(op_w) * kib if op_w else None
        alg, alg_read, alg_write = t.alg_bytes, t.read_bytes, t.write_bytes
        summary.update({
            "copy_kernel": cp_name, "copy_fetch_kib": min(cp_f) if cp_f else None,
            "copy_write_kib": min(cp_w) if cp_w else None, "fetch_scale": f_scale,
            "write_scale": w_scale, "op_fetch_bytes_raw": op_fetch, "op_write_bytes_raw": op_write,
            "op_fetch_bytes": op_fetch * f_scale if op_fetch else None,
            "op_write_bytes": op_write * w_scale if op_write else None,
            "alg_read_bytes": alg_read, "alg_write_bytes": alg_write, "alg_bytes": alg,
        })
        if op_fetch and op_write:
            summary["hbm_bytes_per_dispatch"] = op_fetch * f_scale + op_write * w_scale
            summary["hbm_over_alg"] = summary["hbm_bytes_per_dispatch"] / alg
        if summary.get("op_read_bytes_by_request") and op_write:
            summary["hbm_bytes_by_request"] = summary["op_read_bytes_by_request"] + op_write * w_scale
            summary["by_request_over_alg"] = summary["hbm_bytes_by_request"] / alg
            summary["read_by_request_over_alg_read"] = summary["op_read_bytes_by_request"] / alg_read
        lines = ["# rocprofv3 FETCH_SIZE / WRITE_SIZE, kernel %s, workload %s" % (op_kernel, label),
                 "# commands (from the repository root):",
                 "#   %s" % " ".join(cmds["fetch"]), "#   %s" % " ".join(cmds["write"]),
                 "# counters are KiB per dispatch; the %d-byte streaming-copy probe calibrates them"
                 % COPY_BYTES,
                 "# (scale = known bytes / counted bytes); the minimum over dispatches is used",
                 "# reads by request size (no calibration): %s" % (" ".join(cmds["reqs"]) if "reqs" in cmds
                                                                    else "not taken"), ""]
        for k in ("copy_kernel", "copy_fetch_kib", "copy_write_kib", "fetch_scale", "write_scale",
                  "op_fetch_bytes_raw", "op_write_bytes_raw", "op_fetch_bytes", "op_write_bytes",
                  "alg_read_bytes", "alg_write_bytes", "alg_bytes", "hbm_bytes_per_dispatch",
                  "hbm_over_alg", "copy_read_bytes_by_request", "copy_read_requests",
                  "op_read_bytes_by_request", "op_read_requests", "read_by_request_over_alg_read",
                  "hbm_bytes_by_request", "by_request_over_alg"):
            lines.append("%-24s %s" % (k, summary.get(k)))
        lines += ["", "# machine-readable:", json.dumps({k: summary.get(k) for k in (
            "workload", "kernel", "kernel_sha", "hbm_bytes_per_dispatch", "op_fetch_bytes", "op_write_bytes",
            "alg_bytes", "fetch_scale", "write_scale", "op_read_bytes_by_request", "hbm_bytes_by_request")})]
        text = "\n".join(lines) + "\n"
        open(os.path.join(out, "%s_counters_%s.txt" % (prefix, label)), "w").write(text)
        log(text)

    if "waves" in passes:
        ctrs = args.wave_counters.split(",")
        cmd, d, _ = run_pass("waves", ["--pmc"] + ctrs, args.workload, 3, out, 180)
        rows = counter_rows(d)
        lines = ["# rocprofv3 wave counters, kernel %s, workload %s" % (op_kernel, label),
                 "# command (from the repository root): %s" % " ".join(cmd), ""]
        means = {}
        for c in ctrs:
            name, vals = pick(per_dispatch(rows, c), op_kernel)
            lines.append("%-20s %s" % (c, vals))
            means[c] = sum(vals) / len(vals) if vals else None
        lines.append("")
        lines.append("OccupancyPercent = 400 * sum(SQ_WAVE_CYCLES) / GRBM_GUI_ACTIVE / CUs / 32 "
                     "(resident waves as a share of 32 wave slots per CU); MeanOccupancyPerCU = "
                     "mean resident waves per CU (rocprofv3 derived counters)")
        lines += ["", "# machine-readable (means over the dispatches):", json.dumps({
            "workload": label, "kernel": op_kernel, "kernel_sha": summary["kernel_sha"],
            "mean_occupancy_per_cu": means.get("MeanOccupancyPerCU"),
            "occupancy_percent": means.get("OccupancyPercent")})]
        text = "\n".join(lines) + "\n"
        open(os.path.join(out, "%s_waves_%s.txt" % (prefix, label)), "w").write(text)
        log(text)

    if "bench" in passes:
        if t.family != "op" or args.workload not in W.WORKLOADS:
            raise SystemExit("the bench pass takes an operator workload")
        bench_args = ["--workload", args.workload, "--steps", str(args.bench_steps), "--warmup", str(args.bench_warmup),
                      "--no-also", "--no-variants", "--no-cpu-baseline"]
        cmd, d, json_line = run_pass("bench", ["--kernel-trace", "--stats"], args.workload, 0, out, 900,
                                     bench_args=bench_args)
        rec = json.loads(json_line)
        rows = kernel_stats(d)
        shape = rec["config"]["launch"]
        top = main_instance(rows, op_kernel)
        durs = dispatch_durations(d, top["Name"])
        k, wu = args.bench_steps, args.bench_warmup
        region = durs[wu:wu + k]
        region_avg = sum(region) / len(region)
        lines = ["# rocprofv3 kernel trace over bench.py's run, kernel %s, workload %s" % (op_kernel, label),
                 "# command (from the repository root): %s" % " ".join(cmd),
                 "# kernel source sha256[:16] = %s" % summary["kernel_sha"],
                 "# the workload's launches of %s (rows_per_wave %d), in order: %d warmup, %d in the timed region,"
                 % (op_kernel, shape["rows_per_wave"], wu, k)
                 + " %d event-timed one by one, 10 after a cache flush, %d after the GPU idled;" % (k, k),
                 "# the bench's known-answer checks on the tiny workload use the small-batch template instance"
                 " (rows_per_wave 2), listed on its own line", "",
                 "%-70s %6s %14s %14s %14s" % ("kernel", "calls", "avg_us", "min_us", "max_us")]
        for r in rows:
            lines.append("%-70s %6s %14.2f %14.2f %14.2f" % (
                r["Name"][:70], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3))
        lines += ["", "# the timed region's %d launches in the per-dispatch trace (us):" % len(region),
                  "region_launch_us        %s" % json.dumps([round(x, 2) for x in region]),
                  "region_avg_us           %.2f" % region_avg,
                  "", "# the bench's own figures in the same run (HIP events over the timed region; wall-clock value):",
                  "roofline.kernel_us_mean  %s" % rec["roofline"]["kernel_us_mean"],
                  "kernel_us               %s" % json.dumps(rec["kernel_us"]),
                  "value_gbps              %s" % rec["value"],
                  "", "# machine-readable:", json.dumps({
                      "workload": label, "kernel": op_kernel, "kernel_sha": summary["kernel_sha"],
                      "op_avg_us": round(region_avg, 2), "op_avg_us_all_launches": float(top["AverageNs"]) / 1e3,
                      "op_calls": int(top["Calls"]), "steps": k, "warmup": wu,
                      "bench_kernel_us_mean": rec["roofline"]["kernel_us_mean"]})]
        text = "\n".join(lines) + "\n"
        open(os.path.join(out, "%s_kernel_trace_bench_%s.txt" % (prefix, label)), "w").write(text)
        log(text)

    json.dump(summary, open(os.path.join(out, "summary_%s.json" % label), "w"), indent=1)


if __name__ == "__main__":
    main()
