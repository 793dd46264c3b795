"""Benchmark of the fused q/kv norm-rope-quant-insert operator on one MI355X.

One step = one call of the operator over the whole batch (every q head and kv
row of every token: norm, RoPE, q written back, kv quantized and inserted).
The metric is effective HBM bandwidth: the operator's algorithmic bytes (read
+ written once) divided by the time per step, reported as GB/s, as a fraction
of the 8 TB/s HBM3E peak and as a fraction of a warm device-to-device copy
ceiling measured in the same process.

Order of a run: a known-answer check on the Tiny workload; the headline
workload's inputs drawn on the GPU; the copy ceilings (the "before" set)
measured right after, so that the operator's warmup and timed steps follow a
sustained streaming load, as the ceilings themselves do; W warmup steps; the
K timed steps; then the per-launch, flushed-cache and after-idle passes of the
same workload, the second operator workload, the other workloads and the
neighbouring paths, the "after" ceilings, the known-answer check again and the
CPU baseline.

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
IDLE_S = 1.0


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


def copy_ceilings(torch, probe):
    """The ceilings at 512 MiB and 2 GiB: the runtime's hipMemcpyAsync, the
    probe library's streaming copy and its in-place streaming update (the
    operator rewrites q in place; counted as bytes read + bytes written).  The
    largest rate is the denominator."""
    out = {}
    update = lambda dst, src, nbytes, stream: probe.qkv_prep_probe_update(dst, nbytes, stream)
    for label, fn in (("hipMemcpyAsync", DeviceCopy()), ("probe_copy", probe.qkv_prep_probe_copy),
                      ("probe_update", update)):
        for size in (512 << 20, 2 << 30):
            out["%s_%dMiB" % (label, size >> 20)] = round(copy_rate(torch, fn, size), 1)
    return out


# ----------------------------------------------------------------- timing

def time_region(torch, fn, steps):
    """The timed region: `steps` back-to-back launches bracketed by
    synchronizations, with one HIP event just before the first launch and one
    just after the last, on torch's current stream (the stream the library
    launches on).  Returns (wall seconds, event seconds)."""
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, start.elapsed_time(end) * 1e-3


def time_each(torch, fn, reps):
    """Per-launch durations, each launch between two HIP events."""
    stream = torch.cuda.current_stream()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
    for e0, e1 in events:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) * 1e-3 for e0, e1 in events]


def time_graph(torch, launch, per_graph=100, replays=5):
    """Mean time per launch with the host out of the loop: `per_graph`
    launches captured in one HIP graph (each a prepared call on the capturing
    stream), the graph replayed `replays` times between two HIP events on
    torch's current stream, after one untimed replay."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = launch.on_stream(torch.cuda.current_stream().cuda_stream)
        for _ in range(per_graph):
            captured()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(replays):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e-3 / (per_graph * replays)


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


# ----------------------------------------------------------------- profiles

def profile_record(prefix, kind, label, family):
    """The machine-readable record of a committed rocprofv3 summary
    (profiles/<prefix>_<kind>_<label>.txt), or None when the file is missing
    or was taken on other sources than the current ones of the kernel family."""
    path = os.path.join(ROOT, "profiles", "%s_%s_%s.txt" % (prefix, kind, label))
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
    return rec if rec.get("kernel_sha") == kernel_sha(family) else None


def profile_fields(t, alg_bytes):
    """From the current profiles of target t: HBM bytes per launch (FETCH_SIZE
    and WRITE_SIZE, each scaled by a copy of known size), the mean resident
    waves per CU, and the trace's average launch duration with the fraction
    of peak it gives.  Fields whose summary is missing or stale are None."""
    ctr = profile_record(t.prefix, "counters", t.label, t.family)
    waves = profile_record(t.prefix, "waves", t.label, t.family)
    trace = (profile_record(t.prefix, "kernel_trace_bench", t.label, t.family) or
             profile_record(t.prefix, "kernel_trace", t.label, t.family))
    out = {"traffic": ctr.get("hbm_bytes_per_dispatch") if ctr else None,
           "fetch_bytes": ctr.get("op_fetch_bytes") if ctr else None,
           "write_bytes": ctr.get("op_write_bytes") if ctr else None,
           "waves_per_cu": waves.get("mean_occupancy_per_cu") if waves else None,
           "occupancy_percent": waves.get("occupancy_percent") if waves else None,
           "kernel_us_trace": trace.get("op_avg_us") if trace else None,
           "frac_trace": None}
    if trace and trace.get("op_avg_us"):
        out["frac_trace"] = round(alg_bytes / (trace["op_avg_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)
    return out


# ----------------------------------------------------------------- workloads

def bench_workload(torch, W, qp, probe, name, steps, warmup, ceiling_first):
    """One operator workload: inputs drawn; with ceiling_first, the copy
    ceilings measured right after; W warmup steps; the K timed steps; then a
    per-launch pass, a flushed-cache pass, and a K-step region started after
    the GPU idled for IDLE_S seconds."""
    w = W.WORKLOADS[name]
    log("bench: drawing %s inputs on the GPU" % w.label)
    inp = W.make_inputs(w, device="cuda")
    valid = int(((inp["slot_mapping"] >= 0) &
                 (inp["slot_mapping"] < w.num_blocks * w.block_size)).sum())
    nbytes = W.algorithmic_bytes(w.num_tokens, w.num_heads, valid)
    op = qp.QkvPrep(w.num_heads, block_size=w.block_size, eps=w.eps)
    shape = op.launch_shape(w.num_tokens)
    # checked once; each step is then one C call (qkv_prep_run)
    fn = op.prepare(inp["q"], inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"],
                    inp["slot_mapping"], inp["cache"])
    ceilings = None
    if ceiling_first:
        ceilings = copy_ceilings(torch, probe)
        log("bench: copy ceilings before = %s GB/s" % ceilings)
    log("bench: %s warmup %d" % (w.label, warmup))
    for _ in range(warmup):
        fn()
    log("bench: %s timing %d steps" % (w.label, steps))
    wall, region = time_region(torch, fn, steps)
    each = time_each(torch, fn, steps)
    log("bench: %s cold-cache launches" % w.label)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    cold = time_cold(torch, fn, min(steps, 10), scratch)
    del scratch
    log("bench: %s region after %.1f s idle" % (w.label, IDLE_S))
    torch.cuda.synchronize()
    time.sleep(IDLE_S)
    _, region_idle = time_region(torch, fn, steps)
    res = {
        "workload": "%s %dx%d" % (name, w.num_tokens, w.num_heads),
        "label": "%s_%dx%d" % (name, w.num_tokens, w.num_heads),
        "bytes_per_step": nbytes,
        "wall_s_per_step": wall / steps,
        "kernel_s_mean": region / steps,
        "kernel_s_median": statistics.median(each),
        "kernel_s_min": min(each),
        "kernel_s_p90": p90(each),
        "kernel_s_median_cold": statistics.median(cold),
        "kernel_s_p90_cold": p90(cold),
        "kernel_s_mean_after_idle": region_idle / steps,
        "launch": {"rows_per_wave": shape.rows_per_wave, "waves_per_block": shape.waves_per_block,
                   "convert": shape.convert, "kv_per_wave": shape.kv_per_wave, "grid": shape.grid},
        "valid_slots": valid,
    }
    res["gbps_wall"] = nbytes / res["wall_s_per_step"] / 1e9
    res["gbps_kernel_mean"] = nbytes / res["kernel_s_mean"] / 1e9
    del inp, fn
    torch.cuda.empty_cache()
    return w, res, ceilings


def kernel_us(res):
    return {k: round(res["kernel_s_" + k] * 1e6, 2)
            for k in ("median", "min", "p90", "median_cold", "p90_cold", "mean_after_idle")}


def bench_configs(torch, qp, names, warmup):
    """The other workloads, each after a short sustained streaming load (like
    the headline, which follows its ceiling measurement): the mean launch
    time over a region of back-to-back launches, then per-launch event timings (median,
    min and p90) over as many launches, 200 for the small workloads (Tiny,
    Decode-like) and 30 for the large ones, and the median of 10 launches with
    L2 and the MALL flushed first.  For short kernels the two events around
    each launch add a microsecond or two, which the region does not pay.  The
    small workloads also get a graph-replay mean (100 launches per graph), the
    launch-bound loop with the host taken out."""
    from fp8_kv_cache_amd import probe
    from fp8_kv_cache_amd import variants as V
    out = {}
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    for name in names:
        t = V.target(name)
        log("bench: config %s" % t.label)
        fn = V.setup(t, torch, qp)
        warm_chip(torch, probe)
        for _ in range(warmup):
            fn()
        reps = 200 if t.alg_bytes < (1 << 30) else 30
        _, region = time_region(torch, fn, reps)
        ks = time_each(torch, fn, reps)
        cold = time_cold(torch, fn, 10, scratch)
        graph = time_graph(torch, fn) if reps == 200 else None
        del fn
        torch.cuda.empty_cache()
        med = statistics.median(ks)
        prof = profile_fields(t, t.alg_bytes)
        out[t.label] = {"gbps_region": round(t.alg_bytes * reps / region / 1e9, 1),
                        "gbps_median": round(t.alg_bytes / med / 1e9, 1), "reps": reps,
                        "kernel_us": {"region_mean": round(region / reps * 1e6, 2),
                                      "median": round(med * 1e6, 2), "min": round(min(ks) * 1e6, 2),
                                      "p90": round(p90(ks) * 1e6, 2),
                                      "median_cold": round(statistics.median(cold) * 1e6, 2),
                                      "graph_replay_mean": None if graph is None else round(graph * 1e6, 2)},
                        "bytes_per_launch": t.alg_bytes, "traffic": prof["traffic"],
                        "waves_per_cu": prof["waves_per_cu"]}
    del scratch
    torch.cuda.empty_cache()
    return out


def bench_variants(torch, qp, steps, warmup):
    """The neighbouring paths, each timed like the operator (after a short
    sustained streaming load, then W warmups and K steps): the bf16-store cache
    mode on the Prefill workload (1024-byte slots, no quantization); the cache
    reader gathering every slot of a 4096 x 64-slot cache (262144 rows) to bf16
    and to fp32 as a block-table walk, and to fp32 in a fully random slot order;
    and the MXFP8 norm-quant operator on 16384 x 7168 with the residual add and
    the residual output."""
    from fp8_kv_cache_amd import probe
    from fp8_kv_cache_amd import variants as V
    out = {}
    for name in V.VARIANTS:
        t = V.target(name)
        log("bench: variant %s" % t.label)
        fn = V.setup(t, torch, qp)
        warm_chip(torch, probe)
        for _ in range(warmup):
            fn()
        wall, region = time_region(torch, fn, steps)
        ks = time_each(torch, fn, steps)
        del fn
        torch.cuda.empty_cache()
        mean = region / steps
        roof = {"bound": "hbm", "kernel": t.kernel, "achieved": round(t.alg_bytes / mean / 1e9, 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(t.alg_bytes / mean / 1e9 / PEAK_HBM_GBPS, 4), "bytes_per_launch": t.alg_bytes}
        roof.update(profile_fields(t, t.alg_bytes))
        out[t.label] = {"gbps": round(t.alg_bytes * steps / wall / 1e9, 1),
                        "kernel_us_mean": round(mean * 1e6, 2),
                        "kernel_us_median": round(statistics.median(ks) * 1e6, 2), "roofline": roof}
    return out


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


def cpu_pass(torch, W, name, threads, chunk_tokens=4096, max_tokens=None):
    """The oracle (plain scalar C, OpenMP over tokens) over the workload's
    tokens, chunk by chunk: each chunk's inputs are drawn on the GPU with the
    workload's seed (the same draw the GPU run takes), copied to the host, and
    the oracle is timed around its compute only.  Returns (algorithmic bytes
    of the tokens covered, compute seconds, tokens covered)."""
    import numpy as np
    import oracle
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w, device="cuda")
    T = w.num_tokens if max_tokens is None else min(w.num_tokens, max_tokens)
    pos = inp["positions"].cpu().numpy()
    slots = inp["slot_mapping"].cpu().numpy()
    cs = inp["cos_sin"].cpu().numpy()
    cache = inp["cache"].cpu().numpy()
    qw, kvw = W.as_u16(inp["q_w"]), W.as_u16(inp["kv_w"])
    out = np.zeros((min(chunk_tokens, T), w.num_heads, 512), np.uint16)   # pages touched once
    compute = 0.0
    for t0 in range(0, T, chunk_tokens):
        t1 = min(T, t0 + chunk_tokens)
        q = W.as_u16(inp["q"][t0:t1])
        kv = W.as_u16(inp["kv"][t0:t1])
        o = out[: t1 - t0]
        c0 = time.perf_counter()
        oracle.qkv_prep(q, kv, qw, kvw, pos[t0:t1], cs, slots[t0:t1], cache, w.num_blocks, w.block_size,
                        w.eps, threads, out=o)
        compute += time.perf_counter() - c0
    valid = int(((slots[:T] >= 0) & (slots[:T] < w.num_blocks * w.block_size)).sum())
    del inp
    torch.cuda.empty_cache()
    return W.algorithmic_bytes(T, w.num_heads, valid), compute, T


def cpu_baseline(torch, W, names):
    """The oracle over every token of each named workload on the host cores
    (at most 16 threads), plus a one-thread figure on the first 2048 tokens of
    the first workload.  Throughput uses the same byte formula as the GPU
    figure.  The first workload's figure is the baseline's value."""
    model, usable = host_cpu()
    nth = max(1, min(16, usable))
    per = {}
    for name in names:
        log("bench: cpu baseline %s (%d threads)" % (name, nth))
        nbytes, secs, T = cpu_pass(torch, W, name, nth)
        w = W.WORKLOADS[name]
        per["%s_%dx%d" % (name, w.num_tokens, w.num_heads)] = {
            "gbps": round(nbytes / secs / 1e9, 3), "tokens": T, "compute_s": round(secs, 2)}
    log("bench: cpu baseline, one thread")
    nb1, s1, T1 = cpu_pass(torch, W, names[0], 1, chunk_tokens=2048, max_tokens=2048)
    first = next(iter(per.values()))
    return {"value": first["gbps"], "unit": "GB/s", "cores": nth, "kind": "oracle",
            "sample": "every token of %s, in 4096-token chunks; compute time only" % " and ".join(per),
            "cpu_model": model, "host_cpus": usable, "per_workload": per,
            "value_1_core": round(nb1 / s1 / 1e9, 3),
            "sample_1_core": "first %d tokens of %s" % (T1, names[0])}


# ----------------------------------------------------------------- profile mode

def profile_run(torch, qp, probe, name, launches, copy_bytes=512 << 20, copies=3):
    """A short program for rocprofv3: half a second of sustained streaming
    (the probe's in-place update, so the launches that follow run in the
    chip's warm power state, as the bench's do), then `launches` back-to-back
    launches of one target (the operator on a workload, or a neighbouring
    path), then a few launches of the probe library's streaming copy over a
    buffer of known size (its FETCH_SIZE/WRITE_SIZE calibrate the counters
    against bytes that are known exactly)."""
    from fp8_kv_cache_amd import variants as V
    t = V.target(name)
    fn = V.setup(t, torch, qp)
    torch.cuda.synchronize()
    warm_chip(torch, probe)
    for _ in range(launches):
        fn()
    torch.cuda.synchronize()
    log("profile: %s, %d launches done" % (t.label, launches))
    del fn
    torch.cuda.empty_cache()
    src = torch.ones(copy_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for i in range(copies):
        probe.qkv_prep_probe_copy(dst.data_ptr(), src.data_ptr(), copy_bytes,
                                  torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    log("profile: %d copies of %d bytes done" % (copies, copy_bytes))


# ----------------------------------------------------------------- sweep mode

def warm_chip(torch, probe, seconds=0.5, nbytes=2 << 30):
    """Sustained in-place streaming for about `seconds`, so that what follows
    runs in the chip's warm power state: after a lull, the first ~15 ms of
    sustained streaming run up to 25% slow."""
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            probe.qkv_prep_probe_update(buf.data_ptr(), nbytes, stream)
        torch.cuda.synchronize()
    del buf


def sweep_workload(W, name, size, block_size=0):
    """A named workload, or for size "TxH" a decode-like one of that size:
    positions uniform in [0, 131072), random distinct slots of a cache twice
    the token count.  block_size > 0 re-cuts the cache into blocks of that
    many slots, keeping its slot count (the slot recipe follows the new
    blocks)."""
    import dataclasses
    if not size:
        w = W.WORKLOADS[name]
    else:
        T, H = (int(v) for v in size.lower().split("x"))
        w = W.custom(T, H, seed=11 + T + H, max_position=131072)
    if block_size and block_size != w.block_size:
        slots = w.num_blocks * w.block_size
        if slots % block_size:
            raise ValueError("the cache's %d slots do not split into blocks of %d" % (slots, block_size))
        w = dataclasses.replace(w, block_size=block_size, num_blocks=slots // block_size)
    return w


def parse_shapes(text):
    """'r:b:k,...' (q rows per wavefront, wavefronts per workgroup, kv tokens
    per wavefront) -> a list of forced shapes; '' -> None (every shape)."""
    if not text:
        return None
    out = []
    for item in text.split(","):
        r, b, k = (int(v) for v in item.split(":"))
        out.append(dict(rows_per_wave=r, waves_per_block=b, kv_per_wave=k))
    return out


def sweep_shapes(torch, W, qp, name, size=None, launches=30, rounds=3, only=None, block_size=0):
    """Every forced launch shape of the operator on one workload (rows per
    wavefront 1/2/4 x wavefronts per workgroup 1/2/4/8 x kv tokens per
    wavefront 1/2/4), plus both conversion paths at the heuristic's shape, or
    only the shapes in `only`: the region time of `launches` back-to-back
    launches, best of `rounds` interleaved rounds, with the chip warmed first.
    Every shape computes the same bits (the GPU parity tests check each one);
    this measures only their speed, so the heuristic's choice can be
    re-checked on any machine."""
    from fp8_kv_cache_amd import probe
    w = sweep_workload(W, name, size, block_size)
    name = w.name
    inp = W.make_inputs(w, device="cuda")
    valid = int(((inp["slot_mapping"] >= 0) & (inp["slot_mapping"] < w.num_blocks * w.block_size)).sum())
    nbytes = W.algorithmic_bytes(w.num_tokens, w.num_heads, valid)
    args = (inp["q"], inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"],
            inp["slot_mapping"], inp["cache"])
    heur = qp.QkvPrep(w.num_heads, block_size=w.block_size, eps=w.eps).launch_shape(w.num_tokens)
    if only is None:
        shapes = [dict(rows_per_wave=r, waves_per_block=b, kv_per_wave=k)
                  for r in (1, 2, 4) for b in (1, 2, 4, 8) for k in (1, 2, 4)]
        shapes += [dict(rows_per_wave=heur.rows_per_wave, waves_per_block=heur.waves_per_block,
                        kv_per_wave=heur.kv_per_wave, convert=c) for c in (1, 2)]
    else:
        shapes = list(only)
    ops = [qp.QkvPrep(w.num_heads, block_size=w.block_size, eps=w.eps, **sh) for sh in shapes]
    launches_of = [op.prepare(*args) for op in ops]
    warm_chip(torch, probe)
    best = [float("inf")] * len(shapes)
    for rnd in range(rounds):
        order = range(len(shapes)) if rnd % 2 == 0 else reversed(range(len(shapes)))
        for i in order:
            fn = launches_of[i]
            for _ in range(3):
                fn()
            _, region = time_region(torch, fn, launches)
            best[i] = min(best[i], region / launches)
    rows = sorted(({"shape": sh, "us": round(t * 1e6, 2), "gbps": round(nbytes / t / 1e9, 1)}
                   for sh, t in zip(shapes, best)), key=lambda r: r["us"])
    del inp, args, ops, launches_of
    torch.cuda.empty_cache()
    res = {"mode": "sweep", "workload": "%s %dx%d" % (name, w.num_tokens, w.num_heads),
           "cache": "%d blocks x %d slots" % (w.num_blocks, w.block_size),
           "bytes_per_launch": nbytes, "launches": launches, "rounds": rounds,
           "heuristic": {"rows_per_wave": heur.rows_per_wave, "waves_per_block": heur.waves_per_block,
                         "kv_per_wave": heur.kv_per_wave, "convert": heur.convert},
           "shapes": rows}
    res.update(heuristic_standing(res))
    return res


def heuristic_standing(res):
    """How the heuristic's shape compares with the fastest shape of one sweep
    result: {"heuristic_us", "best_us", "heuristic_over_best"} (the last as
    a fraction, 0 when the heuristic is the fastest), with None for the
    heuristic's time when its shape was not among those swept.  A swept shape
    without a conversion field runs the default conversion path, the one
    the heuristic takes."""
    h = res["heuristic"]
    key = (h["rows_per_wave"], h["waves_per_block"], h["kv_per_wave"])
    best = min(r["us"] for r in res["shapes"])
    mine = [r["us"] for r in res["shapes"]
            if (r["shape"]["rows_per_wave"], r["shape"]["waves_per_block"], r["shape"]["kv_per_wave"]) == key
            and r["shape"].get("convert", h["convert"]) == h["convert"]]
    if not mine:
        return {"heuristic_us": None, "best_us": best, "heuristic_over_best": None}
    return {"heuristic_us": min(mine), "best_us": best, "heuristic_over_best": round(min(mine) / best - 1, 4)}


def sweep_summary(results):
    """One line over a sweep of several sizes: the mean and largest excess
    of the heuristic's shape over the fastest shape, and where the largest
    one falls (sizes whose heuristic shape was not swept are left out)."""
    got = [(r["heuristic_over_best"], r["workload"]) for r in results if r["heuristic_over_best"] is not None]
    if not got:
        return {"mode": "sweep_summary", "sizes": 0}
    worst = max(got)
    return {"mode": "sweep_summary", "sizes": len(got),
            "mean_heuristic_over_best": round(sum(g for g, _ in got) / len(got), 4),
            "max_heuristic_over_best": worst[0], "worst": worst[1]}


# ----------------------------------------------------------------- streams mode

def stream_table(probe):
    """The streams timed by --mode streams: (label, kind, load policy, store
    policy, sleep, lanes per workgroup, chunks per lane, XCD-contiguous order).  Reads, writes,
    copies and in-place updates with the cache-policy bits the kernels choose
    between, the pause before the store that an in-place update was once
    thought to need, the workgroup sizes of the copy and the update, and
    several chunks per lane with all their loads issued first (with 64 lanes,
    several consecutive 1 KiB rows per wavefront: the "several tokens' loads
    in flight" shape), and the copy and the update with each XCD streaming one
    contiguous eighth of the buffer."""
    R, Wr, C, U = probe.READ, probe.WRITE, probe.COPY, probe.UPDATE
    NT, SC1, SC0 = probe.NT, probe.SC1, probe.SC0
    return [
        ("read plain", R, 0, 0, 0, 256, 1, 0),
        ("read nt", R, NT, 0, 0, 256, 1, 0),
        ("read nt sc1", R, NT | SC1, 0, 0, 256, 1, 0),
        ("write plain", Wr, 0, 0, 0, 256, 1, 0),
        ("write nt", Wr, 0, NT, 0, 256, 1, 0),
        ("write sc1", Wr, 0, SC1, 0, 256, 1, 0),
        ("write nt sc1", Wr, 0, NT | SC1, 0, 256, 1, 0),
        ("write sc0 nt sc1", Wr, 0, SC0 | NT | SC1, 0, 256, 1, 0),
        ("copy plain -> plain", C, 0, 0, 0, 256, 1, 0),
        ("copy nt -> nt", C, NT, NT, 0, 256, 1, 0),
        ("copy nt -> nt sc1", C, NT, NT | SC1, 0, 256, 1, 0),
        ("copy nt sc1 -> nt sc1", C, NT | SC1, NT | SC1, 0, 256, 1, 0),
        ("copy nt -> nt sc1, sleep", C, NT, NT | SC1, 1, 256, 1, 0),
        ("copy nt -> nt sc1, 64 lanes", C, NT, NT | SC1, 0, 64, 1, 0),
        ("copy nt -> nt sc1, 1024 lanes", C, NT, NT | SC1, 0, 1024, 1, 0),
        ("copy nt -> nt sc1, 4 chunks per lane", C, NT, NT | SC1, 0, 256, 4, 0),
        ("copy nt -> nt sc1, 16 chunks per lane", C, NT, NT | SC1, 0, 256, 16, 0),
        ("update nt -> nt", U, NT, NT, 0, 64, 1, 0),
        ("update nt -> nt, sleep", U, NT, NT, 1, 64, 1, 0),
        ("update nt -> nt sc1", U, NT, NT | SC1, 0, 64, 1, 0),
        ("update nt -> nt sc1, sleep", U, NT, NT | SC1, 1, 64, 1, 0),
        ("update plain -> plain, sleep", U, 0, 0, 1, 64, 1, 0),
        ("update nt -> nt sc1, sleep, 256 lanes", U, NT, NT | SC1, 1, 256, 1, 0),
        ("update nt -> nt sc1, 2 rows per wavefront", U, NT, NT | SC1, 0, 64, 2, 0),
        ("update nt -> nt sc1, 4 rows per wavefront", U, NT, NT | SC1, 0, 64, 4, 0),
        ("update nt -> nt sc1, 8 rows per wavefront", U, NT, NT | SC1, 0, 64, 8, 0),
        ("update nt -> nt sc1, 16 rows per wavefront", U, NT, NT | SC1, 0, 64, 16, 0),
        ("read nt, 4 chunks per lane", R, NT, 0, 0, 256, 4, 0),
        ("write nt sc1, 4 chunks per lane", Wr, 0, NT | SC1, 0, 256, 4, 0),
        ("copy nt -> nt sc1, 64 lanes, XCD-contiguous", C, NT, NT | SC1, 0, 64, 1, 1),
        ("update nt -> nt sc1, XCD-contiguous", U, NT, NT | SC1, 0, 64, 1, 1),
    ]


def stream_bytes(size):
    """A streams-mode buffer size: MiB, or KiB with a trailing k ("146k"),
    rounded down to whole 16-byte chunks."""
    size = size.strip().lower()
    n = int(size[:-1]) << 10 if size.endswith("k") else int(size) << 20
    if n < 16:
        raise ValueError("a stream needs at least one 16-byte chunk: %r" % size)
    return n // 16 * 16


def sweep_streams(torch, probe, nbytes, launches=20, rounds=4):
    """Every stream of stream_table over `nbytes`-byte buffers: the region
    time of `launches` back-to-back launches, best of `rounds` interleaved
    rounds (alternate rounds in reverse order), after warming the chip.
    Counted traffic: nbytes for a read or a write, 2 * nbytes for a copy or an
    update."""
    table = stream_table(probe)
    src = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")   # chunks XOR to 0, never the key
    dst = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    key = 0x9E3779B9
    stream = torch.cuda.current_stream().cuda_stream

    def launcher(kind, lp, sp, sleep, lanes, depth, xcd):
        if kind == probe.READ:
            d, s_ = sink.data_ptr(), src.data_ptr()
        elif kind == probe.COPY:
            d, s_ = dst.data_ptr(), src.data_ptr()
        else:
            d, s_ = dst.data_ptr(), None
        return lambda: probe.qkv_prep_probe_stream(kind, lp, sp, sleep, lanes, depth, xcd, d, s_, nbytes, key,
                                                   stream)

    fns = [launcher(*row[1:]) for row in table]
    warm_chip(torch, probe)
    best = [float("inf")] * len(table)
    for rnd in range(rounds):
        order = range(len(table)) if rnd % 2 == 0 else reversed(range(len(table)))
        for i in order:
            for _ in range(3):
                fns[i]()
            _, region = time_region(torch, fns[i], launches)
            best[i] = min(best[i], region / launches)
    if int(sink[0].item()) != 0:
        raise RuntimeError("read stream sink was written: the source did not hold zeros")
    rows = []
    for (label, kind, lp, sp, sleep, lanes, depth, xcd), t in zip(table, best):
        traffic = nbytes * (2 if kind in (probe.COPY, probe.UPDATE) else 1)
        rows.append({"stream": label, "kind": kind, "load_policy": lp, "store_policy": sp, "sleep": sleep,
                     "lanes": lanes, "depth": depth, "xcd_order": xcd, "us": round(t * 1e6, 2),
                     "gbps": round(traffic / t / 1e9, 1)})
    del src, dst, sink
    torch.cuda.empty_cache()
    return {"mode": "streams", "bytes": nbytes, "launches": launches, "rounds": rounds, "streams": rows}


# ----------------------------------------------------------------- MXFP8 pattern mode

def mxfp8_pattern(torch, probe, qp, m=None, hidden=None, launches=50, rounds=5):
    """The MXFP8 operator against its own memory access pattern with no
    arithmetic (qkv_prep_probe_mxfp8_pattern) at m x hidden (with the
    residual): the product's prepared launch and the pattern with every
    stream, without the barrier, without the scale words, without the codes,
    and with the two inputs and the residual output only.  Region time of
    `launches` back-to-back launches, best of `rounds` interleaved rounds,
    after warming the chip; each rate counts that variant's own bytes."""
    from fp8_kv_cache_amd import variants as V
    m = m or V.MX_ROWS
    hidden = hidden or V.MX_HIDDEN
    gen = torch.Generator(device="cuda").manual_seed(77)
    x = torch.randn((m, hidden), generator=gen, device="cuda").to(torch.bfloat16)
    r = torch.randn((m, hidden), generator=gen, device="cuda").to(torch.bfloat16)
    gamma = (0.1 * torch.randn(hidden, generator=gen, device="cuda")).to(torch.bfloat16)
    res_out = torch.empty_like(x)
    codes = torch.empty((m, hidden), dtype=torch.uint8, device="cuda")
    nscale = V.mxfp8_scale_bytes(m, hidden)
    scales = torch.empty(nscale, dtype=torch.uint8, device="cuda")
    product = qp.prepare_mxfp8_norm_quant(x, gamma, 1e-6, residual=r, residual_out=res_out, quant_out=codes,
                                          scale_out=scales)
    stream = torch.cuda.current_stream().cuda_stream
    RES, COD, SCA, BAR = probe.MX_RESIDUAL, probe.MX_CODES, probe.MX_SCALES, probe.MX_BARRIER
    mh = m * hidden

    def own_bytes(streams):
        return (2 * mh + (4 * mh if streams & RES else 0) + (mh if streams & COD else 0) +
                (nscale if streams & SCA else 0))

    def pattern(streams):
        return lambda: probe.qkv_prep_probe_mxfp8_pattern(x.data_ptr(), r.data_ptr(), gamma.data_ptr(),
                                                          res_out.data_ptr(), codes.data_ptr(), scales.data_ptr(),
                                                          m, hidden, streams, stream)

    table = [("product kernel", product, own_bytes(RES | COD | SCA) + 2 * hidden)]
    for label, st in (("pattern: every stream, barrier", RES | COD | SCA | BAR),
                      ("pattern: every stream, no barrier", RES | COD | SCA),
                      ("pattern: no scale words", RES | COD | BAR),
                      ("pattern: no codes", RES | SCA | BAR),
                      ("pattern: inputs and residual output only", RES | BAR)):
        table.append((label, pattern(st), own_bytes(st)))
    warm_chip(torch, probe)
    best = [float("inf")] * len(table)
    for rnd in range(rounds):
        order = range(len(table)) if rnd % 2 == 0 else reversed(range(len(table)))
        for i in order:
            fn = table[i][1]
            for _ in range(3):
                fn()
            _, region = time_region(torch, fn, launches)
            best[i] = min(best[i], region / launches)
    rows = [{"variant": label, "us": round(t * 1e6, 2), "bytes": nb, "gbps": round(nb / t / 1e9, 1)}
            for (label, _, nb), t in zip(table, best)]
    out = {"mode": "mxfp8_pattern", "m": m, "hidden": hidden, "launches": launches, "rounds": rounds,
           "rows": rows, "product_rate_over_pattern": round(best[1] / best[0], 4)}
    del product, x, r, gamma, res_out, codes, scales
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------- main

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
    ap.add_argument("--mode", choices=["bench", "profile", "sweep", "streams", "mxfp8-pattern"], default="bench",
                    help="profile: a short fixed program for rocprofv3 (no JSON line); sweep: every "
                         "forced launch shape of the operator on --workload (one JSON line); streams: "
                         "read/write/copy/update streams by cache policy (one JSON line per size); "
                         "mxfp8-pattern: the MXFP8 operator against its own access pattern (--sizes MxH)")
    ap.add_argument("--launches", type=int, default=5)
    ap.add_argument("--sizes", default="",
                    help="sweep mode: comma-separated TxH sizes (decode-like inputs) instead of --workload; "
                         "streams mode: comma-separated buffer sizes in MiB, or KiB with a k suffix "
                         "(default 512,2048)")
    ap.add_argument("--block-sizes", default="",
                    help="sweep mode: comma-separated cache block sizes (slots per block), each timed with "
                         "the workload's slot count kept; default the workload's own")
    ap.add_argument("--shapes", default="",
                    help="sweep mode: only these shapes, as rows_per_wave:waves_per_block:kv_per_wave,...")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0 or args.launches < 1:
        ap.error("--steps and --launches must be at least 1, --warmup at least 0")
    if args.gpus != 1:
        print("bench.py measures one GPU: this operator is per token and needs no collective; "
              "run with --gpus 1 (over N GPUs each would run this kernel on its own share of the "
              "tokens, or of the heads with the kv row replicated).", file=sys.stderr)
        sys.exit(2)

    import torch
    from fp8_kv_cache_amd import probe
    from fp8_kv_cache_amd import qkv_prep as qp
    from fp8_kv_cache_amd import variants as V
    from fp8_kv_cache_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.mode == "profile":
        profile_run(torch, qp, probe, args.workload, args.launches)
        return
    if args.mode == "mxfp8-pattern":
        for size in (args.sizes.split(",") if args.sizes else [""]):
            m, h = (int(v) for v in size.lower().split("x")) if size else (None, None)
            print(json.dumps(mxfp8_pattern(torch, probe, qp, m, h)), flush=True)
        return
    if args.mode == "streams":
        for size in (args.sizes or "512,2048").split(","):
            print(json.dumps(sweep_streams(torch, probe, stream_bytes(size))), flush=True)
        return
    if args.mode == "sweep":
        results = []
        for size in (args.sizes.split(",") if args.sizes else [None]):
            for bs in ([int(v) for v in args.block_sizes.split(",")] if args.block_sizes else [0]):
                results.append(sweep_shapes(torch, W, qp, args.workload, size, only=parse_shapes(args.shapes),
                                            block_size=bs))
                print(json.dumps(results[-1]), flush=True)
        if len(results) > 1:
            print(json.dumps(sweep_summary(results)), flush=True)
        return
    kat_before = known_answer_check(torch, W, qp)
    w, main_res, ceil_before = bench_workload(torch, W, qp, probe, args.workload, args.steps, args.warmup,
                                              ceiling_first=not args.no_ceiling)
    also = None
    if not args.no_also and args.also and args.also != args.workload:
        _, also, _ = bench_workload(torch, W, qp, probe, args.also, args.steps, args.warmup, False)
    others = [n for n in W.WORKLOADS if n not in (args.workload, args.also)]
    configs = None if args.no_variants else bench_configs(torch, qp, others, args.warmup)
    variants = None if args.no_variants else bench_variants(torch, qp, args.steps, args.warmup)
    ceil_after = None if args.no_ceiling else copy_ceilings(torch, probe)
    log("bench: copy ceilings after = %s GB/s" % ceil_after)
    kat_after = known_answer_check(torch, W, qp)
    ceilings = list(ceil_before.values()) + list(ceil_after.values()) if ceil_before else []
    ceiling = max(ceilings) if ceilings else None
    memcpy_ceiling = max(v for k, v in list(ceil_before.items()) + list(ceil_after.items())
                         if k.startswith("hipMemcpy")) if ceil_before else None

    value = main_res["gbps_wall"]
    achieved = main_res["gbps_kernel_mean"]
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "kernel": KERNEL_NAME,
            "kernel_us_mean": round(main_res["kernel_s_mean"] * 1e6, 2),
            "bytes_per_launch": main_res["bytes_per_step"]}
    roof.update(profile_fields(V.target(args.workload), main_res["bytes_per_step"]))
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
        "roofline": roof,
        "kernel_us": kernel_us(main_res),
        "known_answer_before_after": [kat_before, kat_after],
    }
    if also:
        a_roof = profile_fields(V.target(args.also), also["bytes_per_step"])
        out["also"] = {"workload": also["workload"], "value": round(also["gbps_wall"], 1),
                       "kernel_gbps": round(also["gbps_kernel_mean"], 1),
                       "ms_per_step": round(also["wall_s_per_step"] * 1e3, 4),
                       "frac_of_peak": round(also["gbps_wall"] / PEAK_HBM_GBPS, 4),
                       "frac_of_copy": round(also["gbps_wall"] / ceiling, 4) if ceiling else None,
                       "kernel_us_mean": round(also["kernel_s_mean"] * 1e6, 2),
                       "kernel_us": kernel_us(also), "launch": also["launch"],
                       "bytes_per_step": also["bytes_per_step"], "roofline": a_roof}
    if configs:
        out["configs"] = configs
    if variants:
        out["variants"] = variants
    if not args.no_cpu_baseline:
        names = [args.workload] + ([args.also] if also else [])
        out["cpu_baseline"] = cpu_baseline(torch, W, names)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
