"""Host-only checks of bench.py's contract pieces: the one-GPU refusal, the
traffic lookup (current profile summaries are used, stale ones are not) and
the p90 helper."""
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
    for name in ["prefill", "long"] + list(V.VARIANTS):
        t = V.target(name)
        traffic = bench.recorded_traffic(t)
        assert traffic is not None, t.label
        # within a few percent of the algorithmic bytes (the shuffled reader
        # order is the one case with real excess)
        assert 0.99 * t.alg_bytes < traffic < 1.10 * t.alg_bytes, (t.label, traffic / t.alg_bytes)


def test_stale_profile_is_not_reported(tmp_path, monkeypatch):
    t = V.target("prefill")
    prof = tmp_path / "profiles"
    prof.mkdir()
    src = os.path.join(ROOT, "profiles", "%s_counters_%s.txt" % (t.prefix, t.label))
    text = open(src).read()
    (prof / os.path.basename(src)).write_text(text)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic(t) is not None
    (prof / os.path.basename(src)).write_text(text.replace('"kernel_sha": "', '"kernel_sha": "0'))
    assert bench.recorded_traffic(t) is None
    assert bench.recorded_traffic(V.target("tiny")) is None      # no summary at all


def test_p90():
    assert bench.p90([5.0]) == 5.0
    assert bench.p90(list(range(1, 11))) == 10
    assert bench.p90(list(range(100, 0, -1))) == 91


def test_host_cpu():
    model, usable = bench.host_cpu()
    assert isinstance(model, str) and model
    assert usable >= 1
