"""rocprofv3 harness for the qkv_prep kernel.

Runs ``bench.py --mode profile`` (a few launches of the operator on one
workload, then the library's streaming-copy probe over 512 MiB) under
rocprofv3, one pass
per counter group, each as a child process with its own time limit:

  trace   --kernel-trace --stats           per-kernel average duration
  fetch   --pmc FETCH_SIZE                 HBM bytes read per dispatch (KiB)
  write   --pmc WRITE_SIZE                 HBM bytes written per dispatch (KiB)
  waves   --pmc <wave counters>            occupancy

and writes short text summaries (the figures and the exact commands) to the
output directory.  The copy probe's counters against its known byte count
give the scale factor applied to the operator's counters (on gfx950 with this
ROCm, FETCH_SIZE reads about half of the bytes a copy is known to fetch, while
WRITE_SIZE matches).

    python -m fp8_kv_cache_amd.rocprof_harness --workload prefill --out gpurun_out/prof
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
# The sources that define the operator's kernel; the counter summaries carry
# their hash so that a stale summary is never reported as current.
KERNEL_SRCS = [os.path.join(PKG, "csrc", f) for f in
               ("qkv_prep_kernels.hip", "qkvp_device.h", "qkv_prep_internal.h")]
OP_KERNEL = "qkv_prep_kernel"
COPY_KERNEL = "stream_copy"
COPY_BYTES = 512 << 20


def kernel_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, flush=True)


def run_pass(name, rocprof_args, workload, launches, out, timeout):
    d = os.path.join(out, name)
    os.makedirs(d, exist_ok=True)
    rel = os.path.relpath(d, ROOT)
    cmd = ["rocprofv3"] + rocprof_args + ["--output-format", "csv", "-d", rel, "-o", name, "--",
                                          "python3", "bench.py", "--mode", "profile",
                                          "--workload", workload, "--launches", str(launches)]
    log("pass %s: %s" % (name, " ".join(cmd)))
    t0 = time.time()
    res = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=timeout)
    with open(os.path.join(d, "stdout.txt"), "w") as f:
        f.write(res.stdout + "\n--- stderr ---\n" + res.stderr)
    log("pass %s: rc=%d in %.1f s" % (name, res.returncode, time.time() - t0))
    done = "copies of" in res.stderr
    if res.returncode != 0 and not done:
        raise RuntimeError("rocprofv3 pass %s failed (rc %d); see %s" % (name, res.returncode, d))
    return cmd, d


def find_csv(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, d))
    return hits[-1]


def kernel_stats(d):
    rows = list(csv.DictReader(open(find_csv(d, "kernel_stats.csv"))))
    return rows


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
    ap.add_argument("--out", default="gpurun_out/prof")
    ap.add_argument("--launches", type=int, default=5)
    ap.add_argument("--passes", default="trace,fetch,write,waves")
    ap.add_argument("--wave-counters", default="OccupancyPercent,MeanOccupancyPerCU,SQ_WAVES")
    args = ap.parse_args()
    sys.path.insert(0, ROOT)
    from fp8_kv_cache_amd import workloads as W
    w = W.WORKLOADS[args.workload]
    label = "%s_%dx%d" % (w.name, w.num_tokens, w.num_heads)
    out = os.path.abspath(os.path.join(ROOT, args.out))
    os.makedirs(out, exist_ok=True)
    passes = args.passes.split(",")
    summary = {"workload": label, "kernel_sha": kernel_sha()}
    cmds = {}

    if "trace" in passes:
        cmd, d = run_pass("trace", ["--kernel-trace", "--stats"], args.workload, args.launches,
                          out, 300)
        cmds["trace"] = cmd
        rows = kernel_stats(d)
        lines = ["# rocprofv3 kernel trace, workload %s" % label,
                 "# command (from the repository root): %s" % " ".join(cmd),
                 "# kernel source sha256[:16] = %s" % summary["kernel_sha"], "",
                 "%-70s %6s %14s %14s %14s" % ("kernel", "calls", "avg_us", "min_us", "max_us")]
        for r in rows:
            name = r["Name"][:70]
            lines.append("%-70s %6s %14.2f %14.2f %14.2f" % (
                name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3))
            if OP_KERNEL in r["Name"]:
                summary["op_avg_us"] = float(r["AverageNs"]) / 1e3
                summary["op_calls"] = int(r["Calls"])
        text = "\n".join(lines) + "\n"
        open(os.path.join(out, "qkv_prep_kernel_trace_%s.txt" % label), "w").write(text)
        log(text)

    fetch = write = None
    if "fetch" in passes:
        cmd, d = run_pass("fetch", ["--pmc", "FETCH_SIZE"], args.workload, 3, out, 180)
        cmds["fetch"] = cmd
        fetch = per_dispatch(counter_rows(d), "FETCH_SIZE")
    if "write" in passes:
        cmd, d = run_pass("write", ["--pmc", "WRITE_SIZE"], args.workload, 3, out, 180)
        cmds["write"] = cmd
        write = per_dispatch(counter_rows(d), "WRITE_SIZE")
    if fetch is not None and write is not None:
        op_name, op_f = pick(fetch, OP_KERNEL)
        _, op_w = pick(write, OP_KERNEL)
        cp_name, cp_f = pick(fetch, COPY_KERNEL)
        _, cp_w = pick(write, COPY_KERNEL)
        kib = 1024.0
        # The counters report KiB per dispatch; the copy moves COPY_BYTES each
        # way, which calibrates them.
        f_scale = COPY_BYTES / (min(cp_f) * kib) if cp_f else 1.0
        w_scale = COPY_BYTES / (min(cp_w) * kib) if cp_w else 1.0
        op_fetch = min(op_f) * kib if op_f else None
        op_write = min(op_w) * kib if op_w else None
        valid = w.num_tokens  # every workload but tiny fills a slot per token
        alg = W.algorithmic_bytes(w.num_tokens, w.num_heads, valid)
        alg_read = w.num_tokens * (1024 * w.num_heads + 1024 + 16 + 256) + 2048
        alg_write = w.num_tokens * 1024 * w.num_heads + 584 * valid
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
        lines = ["# rocprofv3 FETCH_SIZE / WRITE_SIZE, workload %s" % label,
                 "# commands (from the repository root):",
                 "#   %s" % " ".join(cmds["fetch"]), "#   %s" % " ".join(cmds["write"]),
                 "# counters are KiB per dispatch; the %d-byte streaming-copy probe calibrates them"
                 % COPY_BYTES,
                 "# (scale = known bytes / counted bytes); the minimum over dispatches is used", ""]
        for k in ("copy_kernel", "copy_fetch_kib", "copy_write_kib", "fetch_scale", "write_scale",
                  "op_fetch_bytes_raw", "op_write_bytes_raw", "op_fetch_bytes", "op_write_bytes",
                  "alg_read_bytes", "alg_write_bytes", "alg_bytes", "hbm_bytes_per_dispatch",
                  "hbm_over_alg"):
            lines.append("%-24s %s" % (k, summary.get(k)))
        lines += ["", "# machine-readable:", json.dumps({k: summary.get(k) for k in (
            "workload", "kernel_sha", "hbm_bytes_per_dispatch", "op_fetch_bytes", "op_write_bytes",
            "alg_bytes", "fetch_scale", "write_scale")})]
        text = "\n".join(lines) + "\n"
        open(os.path.join(out, "qkv_prep_counters_%s.txt" % label), "w").write(text)
        log(text)

    if "waves" in passes:
        ctrs = args.wave_counters.split(",")
        cmd, d = run_pass("waves", ["--pmc"] + ctrs, args.workload, 3, out, 180)
        rows = counter_rows(d)
        lines = ["# rocprofv3 wave counters, workload %s" % label,
                 "# command (from the repository root): %s" % " ".join(cmd), ""]
        for c in ctrs:
            name, vals = pick(per_dispatch(rows, c), OP_KERNEL)
            lines.append("%-20s %s" % (c, vals))
        lines.append("")
        lines.append("OccupancyPercent = 400 * sum(SQ_WAVE_CYCLES) / GRBM_GUI_ACTIVE / CUs / 32 "
                     "(resident waves as a share of 32 wave slots per CU); MeanOccupancyPerCU = "
                     "mean resident waves per CU (rocprofv3 derived counters)")
        text = "\n".join(lines) + "\n"
        open(os.path.join(out, "qkv_prep_waves_%s.txt" % label), "w").write(text)
        log(text)

    json.dump(summary, open(os.path.join(out, "summary_%s.json" % label), "w"), indent=1)


if __name__ == "__main__":
    main()
