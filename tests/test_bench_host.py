"""Host-only checks of bench.py's contract pieces: the one-GPU refusal, the
profile lookup (current rocprofv3 summaries are used, stale ones are not), the
p90 helper, and the sweep mode's shape list and heuristic-against-best
report."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from fp8_kv_cache_amd import variants as V  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


@pytest.mark.parametrize("flags", [["--steps", "0"], ["--warmup", "-1"], ["--launches", "0"]])
def test_bad_counts_are_refused(flags):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + flags,
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2 and "at least" in res.stderr and res.stdout == ""


def test_committed_profiles_are_current_for_every_target():
    # Every measured target has a current counter summary whose HBM bytes are
    # within a few percent of the algorithmic bytes (the shuffled reader order
    # is the one case with real excess); the headline pair also has current
    # occupancy and timed-region trace summaries, so the bench line carries
    # FETCH/WRITE bytes, waves per CU and a trace-derived fraction of peak.
    for name in ["prefill", "long"] + list(V.VARIANTS):
        t = V.target(name)
        f = bench.profile_fields(t, t.alg_bytes)
        assert f["traffic"] is not None, t.label
        assert 0.99 * t.alg_bytes < f["traffic"] < 1.10 * t.alg_bytes, (t.label, f["traffic"] / t.alg_bytes)
        assert abs(f["fetch_bytes"] + f["write_bytes"] - f["traffic"]) < 1e-6 * f["traffic"]
        assert f["waves_per_cu"] is not None and 0 < f["waves_per_cu"] <= 32, t.label
        assert f["kernel_us_trace"] is not None and 0 < f["frac_trace"] < 1, t.label
    for name in ("prefill", "long"):
        t = V.target(name)
        assert bench.profile_record(t.prefix, "kernel_trace_bench", t.label, t.family) is not None, name


def test_stale_profile_is_not_reported(tmp_path, monkeypatch):
    t = V.target("prefill")
    prof = tmp_path / "profiles"
    prof.mkdir()
    src = os.path.join(ROOT, "profiles", "%s_counters_%s.txt" % (t.prefix, t.label))
    text = open(src).read()
    (prof / os.path.basename(src)).write_text(text)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profile_fields(t, t.alg_bytes)["traffic"] is not None
    (prof / os.path.basename(src)).write_text(text.replace('"kernel_sha": "', '"kernel_sha": "0'))
    assert bench.profile_fields(t, t.alg_bytes)["traffic"] is None
    assert bench.profile_fields(V.target("tiny"), 1)["traffic"] is None      # no summary at all


def test_p90():
    assert bench.p90([5.0]) == 5.0
    assert bench.p90(list(range(1, 11))) == 10
    assert bench.p90(list(range(100, 0, -1))) == 91


def test_host_cpu():
    model, usable = bench.host_cpu()
    assert isinstance(model, str) and model
    assert usable >= 1


def test_sweep_shape_list():
    assert bench.parse_shapes("") is None
    assert bench.parse_shapes("1:1:4,2:8:1") == [dict(rows_per_wave=1, waves_per_block=1, kv_per_wave=4),
                                                  dict(rows_per_wave=2, waves_per_block=8, kv_per_wave=1)]
    with pytest.raises(ValueError):
        bench.parse_shapes("1:1")


def _sweep_result(workload, heur, times):
    rows = [{"shape": dict(zip(("rows_per_wave", "waves_per_block", "kv_per_wave"), k), **extra), "us": us}
            for (k, extra), us in times]
    return {"workload": workload, "heuristic": dict(zip(("rows_per_wave", "waves_per_block", "kv_per_wave"), heur),
                                                   convert=2), "shapes": rows}


def test_sweep_reports_the_heuristic_against_the_fastest_shape():
    r = _sweep_result("custom 8192x3", (1, 1, 2), [(((1, 1, 2), {}), 12.6), (((2, 1, 1), {}), 15.3),
                                                   (((1, 1, 2), {"convert": 1}), 12.0)])
    # the conversion-1 run of the same shape is not the heuristic's launch
    assert bench.heuristic_standing(r) == {"heuristic_us": 12.6, "best_us": 12.0,
                                           "heuristic_over_best": round(12.6 / 12.0 - 1, 4)}
    r2 = _sweep_result("custom 4096x8", (2, 2, 2), [(((2, 2, 2), {"convert": 2}), 13.5), (((1, 1, 4), {}), 14.2)])
    assert bench.heuristic_standing(r2)["heuristic_over_best"] == 0
    r3 = _sweep_result("custom 16x8", (2, 1, 1), [(((1, 1, 4), {}), 5.0)])
    assert bench.heuristic_standing(r3) == {"heuristic_us": None, "best_us": 5.0, "heuristic_over_best": None}
    for x in (r, r2, r3):
        x.update(bench.heuristic_standing(x))
    s = bench.sweep_summary([r, r2, r3])
    assert s["sizes"] == 2 and s["worst"] == "custom 8192x3"
    assert s["max_heuristic_over_best"] == r["heuristic_over_best"]
    assert s["mean_heuristic_over_best"] == round(r["heuristic_over_best"] / 2, 4)
    assert bench.sweep_summary([r3]) == {"mode": "sweep_summary", "sizes": 0}


def test_sweep_block_sizes_keep_the_slot_count():
    from fp8_kv_cache_amd import workloads as W
    for name in ("prefill", "decode", "long"):
        base = W.WORKLOADS[name]
        for bs in (16, 64, 256):
            w = bench.sweep_workload(W, name, None, bs)
            assert w.block_size == bs and w.num_blocks * bs == base.num_blocks * base.block_size
            assert (w.num_tokens, w.num_heads, w.slots, w.positions) == \
                (base.num_tokens, base.num_heads, base.slots, base.positions)
    assert bench.sweep_workload(W, "prefill", None, 0) == W.WORKLOADS["prefill"]
    with pytest.raises(ValueError):
        bench.sweep_workload(W, "tiny", None, 512)            # 256 slots do not split into 512
    w = bench.sweep_workload(W, "prefill", "1000x8", 16)
    assert w.block_size == 16 and w.num_tokens == 1000


def test_streams_table_holds_only_combinations_the_probe_accepts():
    # With zero bytes the probe checks every argument and launches nothing.
    from fp8_kv_cache_amd import probe
    lib = probe.library()
    table = bench.stream_table(probe)
    assert len({row[0] for row in table}) == len(table)
    for label, kind, lp, sp, sleep, lanes, depth, xcd in table:
        src = None if kind in (probe.WRITE, probe.UPDATE) else 1 << 30
        assert lib.qkv_prep_probe_stream(kind, lp, sp, sleep, lanes, depth, xcd, 1 << 20, src, 0, 0, None) == 0, label
    # the MXFP8 pattern's stream sets, with every buffer given
    for streams in (1 | 2 | 4 | 8, 1 | 2 | 4, 1 | 2 | 8, 1 | 4 | 8, 1 | 8):
        assert lib.qkv_prep_probe_mxfp8_pattern(1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20, 6 << 20, 0, 7168,
                                                streams, None) == 0


def test_stream_sizes():
    assert bench.stream_bytes("512") == 512 << 20
    assert bench.stream_bytes("146k") == 146 << 10
    assert bench.stream_bytes(" 1K ") == 1024
    with pytest.raises(ValueError):
        bench.stream_bytes("0k")
