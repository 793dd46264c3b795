"""Benchmark of the fused q/kv norm-rope-quant-insert operator on one MI355X.

One step = one call of the operator over the whole batch (every q head and kv
row of every token: norm, RoPE, q written back, kv quantized and inserted).
The metric is effective HBM bandwidth: the operator's algorithmic bytes (read
+ written once) divided by the time per step, reported as GB/s, as a fraction
of the 8 TB/s HBM3E peak and as a fraction of a warm device-to-device copy
ceiling measured in the same process.

Prints ONE JSON line.  ``value`` is the Prefill workload (32768 tokens x 64
heads); the Long workload (131072 x 128) is reported under ``also``.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-also]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective HBM GB/s & % of warm copy ceiling, tokens×heads 32768×64 / 131072×128"
PEAK_HBM_GBPS = 8000.0
KERNEL_NAME = "qkv_prep_kernel"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- copy ceiling

class DeviceCopy:
    """hipMemcpyAsync device-to-device through the HIP runtime torch loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_int, ctypes.c_void_p]
        self.hip.hipMemcpyAsync.restype = ctypes.c_int

    def __call__(self, dst, src, nbytes, stream):
        rc = self.hip.hipMemcpyAsync(dst, src, nbytes, 3, stream)   # 3 = device to device
        if rc != 0:
            raise RuntimeError("hipMemcpyAsync failed: %d" % rc)


def copy_rate(torch, copier, size_bytes, reps=20, max_rounds=12):
    """Warm D2D copy rate, counted as 2 x size / time (read + write).  Repeats
    rounds of `reps` copies until three consecutive round medians agree within
    0.5%, and returns the best round median."""
    src = torch.empty(size_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    for _ in range(10):
        copier(dst.data_ptr(), src.data_ptr(), size_bytes, h)
    torch.cuda.synchronize()
    medians = []
    for _ in range(max_rounds):
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            copier(dst.data_ptr(), src.data_ptr(), size_bytes, h)
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        medians.append(statistics.median(times))
        if len(medians) >= 3:
            last = medians[-3:]
            if (max(last) - min(last)) / min(last) < 0.005:
                break
    del src, dst
    return 2.0 * size_bytes / min(medians) / 1e9


def copy_ceilings(torch, qp):
    """The ceilings at 512 MiB and 2 GiB: the runtime's hipMemcpyAsync, the
    library's streaming-copy probe and its in-place streaming-update probe (the
    operator rewrites q in place; counted as bytes read + bytes written).  The
    largest rate is the denominator."""
    out = {}
    update = lambda dst, src, nbytes, stream: qp.qkv_prep_probe_update(dst, nbytes, stream)
    for label, fn in (("hipMemcpyAsync", DeviceCopy()), ("probe_copy", qp.qkv_prep_probe_copy),
                      ("probe_update", update)):
        for size in (512 << 20, 2 << 30):
            out["%s_%dMiB" % (label, size >> 20)] = round(copy_rate(torch, fn, size), 1)
    return out


# ----------------------------------------------------------------- one workload

def time_launches(torch, fn, steps):
    """The timed region: `steps` back-to-back launches bracketed by
    synchronizations, with one HIP event just before the first launch and one
    just after the last, on torch's current stream (the stream the library
    launches on).  Returns the per-launch durations of a second pass of as many
    launches, each between two events (for the median, minimum and p90), the
    wall time of the timed region, and its event time (for the mean launch
    duration over the timed region)."""
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region = start.elapsed_time(end) * 1e-3
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
    for e0, e1 in events:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) * 1e-3 for e0, e1 in events], wall, region


def time_cold(torch, fn, reps, scratch):
    """Per-launch HIP-event durations with L2 and the MALL flushed before each
    launch: a 1 GiB scratch write, on the same stream and outside the events."""
    stream = torch.cuda.current_stream()
    out = []
    for k in range(reps):
        scratch.fill_(k & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        out.append((e0, e1))
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) * 1e-3 for e0, e1 in out]


def p90(xs):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(0.9 * len(xs)))]


def bench_variants(torch, qp, steps, warmup):
    """The neighbouring paths, each timed like the operator: the bf16-store cache
    mode on the Prefill workload (1024-byte slots, no quantization); the cache
    reader gathering every slot of a 4096 x 64-slot cache (262144 rows) to bf16
    and to fp32 as a block-table walk, and to fp32 in a fully random slot order;
    and the MXFP8 norm-quant operator on 16384 x 7168 with the residual add and
    the residual output."""
    from fp8_kv_cache_amd import variants as V
    out = {}
    for name in V.VARIANTS:
        t = V.target(name)
        log("bench: variant %s" % t.label)
        fn = V.setup(t, torch, qp)
        for _ in range(warmup):
            fn()
        ks, wall, region = time_launches(torch, fn, steps)
        del fn
        torch.cuda.empty_cache()
        mean = region / steps
        out[t.label] = {
            "gbps": round(t.alg_bytes * steps / wall / 1e9, 1),
            "kernel_us_mean": round(mean * 1e6, 2),
            "kernel_us_median": round(statistics.median(ks) * 1e6, 2),
            "roofline": {"bound": "hbm", "kernel": t.kernel, "achieved": round(t.alg_bytes / mean / 1e9, 1),
                         "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(t.alg_bytes / mean / 1e9 / PEAK_HBM_GBPS, 4),
                         "traffic": recorded_traffic(t), "bytes_per_launch": t.alg_bytes},
        }
    return out


def bench_configs(torch, W, qp, names, warmup):
    """The other workloads, event-timed per launch: median, min and p90 over
    200 launches for the small ones (Tiny, Decode-like) and 30 for the large
    ones, plus the median of 10 launches with L2 and the MALL flushed first."""
    from fp8_kv_cache_amd import variants as V
    out = {}
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    for name in names:
        t = V.target(name)
        log("bench: config %s" % t.label)
        fn = V.setup(t, torch, qp)
        for _ in range(warmup):
            fn()
        reps = 200 if t.alg_bytes < (1 << 30) else 30
        ks, _, _ = time_launches(torch, fn, reps)
        cold = time_cold(torch, fn, 10, scratch)
        del fn
        torch.cuda.empty_cache()
        med = statistics.median(ks)
        out[t.label] = {"gbps_median": round(t.alg_bytes / med / 1e9, 1), "reps": reps,
                        "kernel_us": {"median": round(med * 1e6, 2), "min": round(min(ks) * 1e6, 2),
                                      "p90": round(p90(ks) * 1e6, 2),
                                      "median_cold": round(statistics.median(cold) * 1e6, 2)},
                        "bytes_per_launch": t.alg_bytes}
    del scratch
    torch.cuda.empty_cache()
    return out


def bench_workload(torch, W, qp, name, steps, warmup):
    w = W.WORKLOADS[name]
    log("bench: drawing %s inputs on the GPU" % w.label)
    inp = W.make_inputs(w, device="cuda")
    valid = int(((inp["slot_mapping"] >= 0) &
                 (inp["slot_mapping"] < w.num_blocks * w.block_size)).sum())
    nbytes = W.algorithmic_bytes(w.num_tokens, w.num_heads, valid)
    op = qp.QkvPrep(w.num_heads, block_size=w.block_size, eps=w.eps)
    shape = op.launch_shape(w.num_tokens)
    args = (inp["q"], inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"],
            inp["slot_mapping"], inp["cache"])
    log("bench: %s warmup %d" % (w.label, warmup))
    for _ in range(warmup):
        op(*args)
    torch.cuda.synchronize()
    log("bench: %s timing %d steps" % (w.label, steps))
    kernel_s, wall, region = time_launches(torch, lambda: op(*args), steps)
    log("bench: %s cold-cache launches" % w.label)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    cold_s = time_cold(torch, lambda: op(*args), min(steps, 10), scratch)
    del scratch
    res = {
        "workload": "%s %dx%d" % (name, w.num_tokens, w.num_heads),
        "bytes_per_step": nbytes,
        "wall_s_per_step": wall / steps,
        "kernel_s_mean": region / steps,
        "kernel_s_median": statistics.median(kernel_s),
        "kernel_s_min": min(kernel_s),
        "kernel_s_p90": p90(kernel_s),
        "kernel_s_median_cold": statistics.median(cold_s),
        "kernel_s_p90_cold": p90(cold_s),
        "launch": {"rows_per_wave": shape.rows_per_wave, "waves_per_block": shape.waves_per_block,
                   "convert": shape.convert, "grid": shape.grid},
        "valid_slots": valid,
    }
    res["gbps_wall"] = nbytes / res["wall_s_per_step"] / 1e9
    res["gbps_kernel_mean"] = nbytes / res["kernel_s_mean"] / 1e9
    res["gbps_kernel_median"] = nbytes / res["kernel_s_median"] / 1e9
    del inp, args
    torch.cuda.empty_cache()
    return w, res


def known_answer_check(torch, W, qp):
    """Tiny workload on the device vs the oracle, bit for bit (run before and
    after the measurement so a device that misbehaves cannot go unnoticed)."""
    import numpy as np
    import oracle
    w = W.WORKLOADS["tiny"]
    inp = W.make_inputs(w, device="cuda")
    q0 = W.as_u16(inp["q"])
    cache = inp["cache"].cpu().numpy().copy()
    qp.QkvPrep(w.num_heads, block_size=w.block_size, eps=w.eps)(
        inp["q"], inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"],
        inp["slot_mapping"], inp["cache"])
    torch.cuda.synchronize()
    want_q = oracle.qkv_prep(q0, W.as_u16(inp["kv"]), W.as_u16(inp["q_w"]), W.as_u16(inp["kv_w"]),
                             inp["positions"].cpu().numpy(), inp["cos_sin"].cpu().numpy(),
                             inp["slot_mapping"].cpu().numpy(), cache, w.num_blocks,
                             w.block_size, w.eps)
    return bool(np.array_equal(W.as_u16(inp["q"]), want_q) and
                np.array_equal(inp["cache"].cpu().numpy(), cache))


# ----------------------------------------------------------------- CPU baseline

def host_cpu():
    """The host's CPU model (first `model name` of /proc/cpuinfo) and the
    number of CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return model, usable


def cpu_baseline(torch, W, name, target_s=12.0, sample_tokens=4096):
    """The oracle (plain scalar C, OpenMP over tokens) on a bounded sample of
    the same workload: its first `sample_tokens` tokens, passed over
    repeatedly until about target_s seconds of CPU work.  Throughput uses the
    same byte formula as the GPU figure.  The output buffer is allocated and
    touched once, so the timed passes are the oracle's compute and memory
    traffic only."""
    import numpy as np
    import oracle
    w = W.WORKLOADS[name]
    nth = max(1, min(16, host_cpu()[1]))        # at most 16 threads
    n = min(w.num_tokens, sample_tokens)
    sub = W.Workload(w.name, n, w.num_heads, w.max_position, w.num_blocks, w.block_size,
                     w.positions, w.slots, w.seed, num_seqs=max(1, n * w.num_seqs // w.num_tokens),
                     outlier_frac=w.outlier_frac)
    inp = W.make_inputs(sub, device="cuda")
    q = W.as_u16(inp["q"])
    kv = W.as_u16(inp["kv"])
    qw, kvw = W.as_u16(inp["q_w"]), W.as_u16(inp["kv_w"])
    pos = inp["positions"].cpu().numpy()
    cs = inp["cos_sin"].cpu().numpy()
    slots = inp["slot_mapping"].cpu().numpy()
    cache = inp["cache"].cpu().numpy()
    valid = int(((slots >= 0) & (slots < w.num_blocks * w.block_size)).sum())
    nbytes = W.algorithmic_bytes(n, w.num_heads, valid)
    out = np.empty_like(q)
    out.fill(0)                       # touch the pages once, outside the timed passes

    def passes(threads, budget):
        done, t0 = 0, time.perf_counter()
        while True:
            oracle.qkv_prep(q, kv, qw, kvw, pos, cs, slots, cache, w.num_blocks, w.block_size,
                            w.eps, threads, out=out)
            done += 1
            dt = time.perf_counter() - t0
            if dt >= budget:
                return done, dt

    k, dt = passes(nth, target_s)
    k1, dt1 = passes(1, 2.0)
    model, usable = host_cpu()
    return {"value": round(nbytes * k / dt / 1e9, 3), "unit": "GB/s", "cores": nth,
            "kind": "oracle", "cpu_model": model, "host_cpus": usable,
            "sample": "first %d of %d tokens of %s %dx%d, %d passes in %.1f s" % (
                n, w.num_tokens, w.name, w.num_tokens, w.num_heads, k, dt),
            "value_1_core": round(nbytes * k1 / dt1 / 1e9, 3)}


# ----------------------------------------------------------------- counters

def recorded_traffic(t):
    """HBM bytes per dispatch of target t from the committed rocprofv3 counter
    summary, if it was taken on the current source of t's kernel (else None)."""
    path = os.path.join(ROOT, "profiles", "%s_counters_%s.txt" % (t.prefix, t.label))
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("{"):
                rec = json.loads(line)
    if not rec:
        return None
    from fp8_kv_cache_amd.rocprof_harness import kernel_sha
    if rec.get("kernel_sha") != kernel_sha(t.family):
        return None
    return rec.get("hbm_bytes_per_dispatch")


# ----------------------------------------------------------------- main

def profile_run(torch, qp, name, launches, copy_bytes=512 << 20, copies=3):
    """A short program for rocprofv3: a few launches of one target (the
    operator on a workload, or a neighbouring path), then a few launches of the
    library's streaming-copy probe over a buffer of known size (its
    FETCH_SIZE/WRITE_SIZE calibrate the counters against bytes that are known
    exactly)."""
    from fp8_kv_cache_amd import variants as V
    t = V.target(name)
    fn = V.setup(t, torch, qp)
    torch.cuda.synchronize()
    for i in range(launches):
        fn()
        torch.cuda.synchronize()
        log("profile: %s launch %d done" % (t.label, i))
    del fn
    torch.cuda.empty_cache()
    src = torch.ones(copy_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for i in range(copies):
        qp.qkv_prep_probe_copy(dst.data_ptr(), src.data_ptr(), copy_bytes,
                               torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    log("profile: %d copies of %d bytes done" % (copies, copy_bytes))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill",
                    help="an operator workload; in profile mode also a variant target "
                         "(bf16store_prefill, gather_bf16, gather_f32, gather_f32_shuffled, mxfp8)")
    ap.add_argument("--also", default="long")
    ap.add_argument("--no-also", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--mode", choices=["bench", "profile"], default="bench",
                    help="profile: a short fixed program for rocprofv3 (no JSON line)")
    ap.add_argument("--launches", type=int, default=5)
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0 or args.launches < 1:
        ap.error("--steps and --launches must be at least 1, --warmup at least 0")
    if args.gpus != 1:
        print("bench.py measures one GPU: this operator is per token and needs no collective; "
              "run with --gpus 1 (see the design notes for how it would shard).", file=sys.stderr)
        sys.exit(2)

    import torch
    from fp8_kv_cache_amd import qkv_prep as qp
    from fp8_kv_cache_amd import variants as V
    from fp8_kv_cache_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.mode == "profile":
        profile_run(torch, qp, args.workload, args.launches)
        return
    kat_before = known_answer_check(torch, W, qp)
    ceil_before = None if args.no_ceiling else copy_ceilings(torch, qp)
    log("bench: copy ceilings before = %s GB/s" % ceil_before)
    w, main_res = bench_workload(torch, W, qp, args.workload, args.steps, args.warmup)
    also = None
    if not args.no_also and args.also and args.also != args.workload:
        _, also = bench_workload(torch, W, qp, args.also, args.steps, args.warmup)
    others = [n for n in W.WORKLOADS if n not in (args.workload, args.also)]
    configs = None if args.no_variants else bench_configs(torch, W, qp, others, args.warmup)
    variants = None if args.no_variants else bench_variants(torch, qp, args.steps, args.warmup)
    ceil_after = None if args.no_ceiling else copy_ceilings(torch, qp)
    log("bench: copy ceilings after = %s GB/s" % ceil_after)
    kat_after = known_answer_check(torch, W, qp)
    ceiling = max(list(ceil_before.values()) + list(ceil_after.values())) if ceil_before else None
    memcpy_ceiling = max(v for k, v in list(ceil_before.items()) + list(ceil_after.items())
                         if k.startswith("hipMemcpy")) if ceil_before else None

    value = main_res["gbps_wall"]
    achieved = main_res["gbps_kernel_mean"]
    traffic = recorded_traffic(V.target(args.workload))
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["wall_s_per_step"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": main_res["workload"], "tokens": w.num_tokens, "heads": w.num_heads,
                   "head_dim": 512, "io": "bf16 q/kv in, bf16 q out in place, fp8 e4m3 + ue8m0 cache",
                   "cache": "%d blocks x %d slots x 584 B" % (w.num_blocks, w.block_size),
                   "launch": main_res["launch"]},
        "frac_of_peak": round(value / PEAK_HBM_GBPS, 4),
        "copy_ceiling_gbps": round(ceiling, 1) if ceiling else None,
        "copy_ceilings_before_after": [ceil_before, ceil_after],
        "frac_of_copy": round(value / ceiling, 4) if ceiling else None,
        "frac_of_hipmemcpy": round(value / memcpy_ceiling, 4) if memcpy_ceiling else None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "kernel": KERNEL_NAME,
                     "kernel_us_mean": round(main_res["kernel_s_mean"] * 1e6, 2),
                     "bytes_per_launch": main_res["bytes_per_step"]},
        "kernel_us": {k: round(main_res["kernel_s_" + k] * 1e6, 2)
                      for k in ("median", "min", "p90", "median_cold", "p90_cold")},
        "known_answer_before_after": [kat_before, kat_after],
    }
    if also:
        out["also"] = {"workload": also["workload"], "value": round(also["gbps_wall"], 1),
                       "kernel_gbps": round(also["gbps_kernel_mean"], 1),
                       "ms_per_step": round(also["wall_s_per_step"] * 1e3, 4),
                       "frac_of_peak": round(also["gbps_wall"] / PEAK_HBM_GBPS, 4),
                       "frac_of_copy": round(also["gbps_wall"] / ceiling, 4) if ceiling else None,
                       "kernel_us": {k: round(also["kernel_s_" + k] * 1e6, 2)
                                     for k in ("median", "min", "p90", "median_cold", "p90_cold")},
                       "launch": also["launch"], "bytes_per_step": also["bytes_per_step"],
                       "traffic": recorded_traffic(V.target(args.also))}
    if configs:
        out["configs"] = configs
    if variants:
        out["variants"] = variants
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(torch, W, args.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
