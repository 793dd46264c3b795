"""The two environment switches of the C library, read by qkv_prep_create:
QKV_PREP_SYNC=1 (every call waits for its stream, so a device error is
reported by the call that caused it) and QKV_PREP_LOG=1 (the handle prints its
launch shape to stderr whenever it changes).  A child process runs with both
set; its results must equal, byte for byte, the same calls made here without
them, and its log must hold exactly one line per change of launch shape."""
import json
import os
import re
import subprocess
import sys

import pytest

from fp8_kv_cache_amd import qkv_prep as qp

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
H = 64
# Token counts in call order, all on one handle: 16 tokens (1024 q rows) take
# two heads per wavefront and one kv token per kv wavefront, 2048 tokens (2^17
# q rows) one row per wavefront and four kv tokens; so the shape changes at
# the third call and back at the fifth, and the repeats keep it.
CALLS = [16, 16, 2048, 2048, 16]

# Runs CALLS on one handle and prints one JSON line per call with the hashes
# of q and the cache after it.  The same code runs here (flags unset) and in
# the child (flags set).
PROGRAM = r"""
import hashlib, json, sys
sys.path.insert(0, %(root)r)
import torch
from fp8_kv_cache_amd import qkv_prep as qp
from fp8_kv_cache_amd import workloads as W
op = qp.QkvPrep(%(heads)d, block_size=64, eps=1e-6)
for T in %(calls)r:
    w = W.custom(T, %(heads)d, seed=T)
    inp = W.make_inputs(w, device="cuda")
    op(inp["q"], inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"], inp["slot_mapping"],
       inp["cache"])
    torch.cuda.synchronize()
    digest = lambda t: hashlib.sha256(t.cpu().numpy().tobytes()).hexdigest()
    print(json.dumps({"T": T, "q": digest(inp["q"].view(torch.int16)), "cache": digest(inp["cache"])}),
          flush=True)
""" % {"root": ROOT, "heads": H, "calls": CALLS}


def run(env):
    res = subprocess.run([sys.executable, "-c", PROGRAM], env=env, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-3000:]
    return [json.loads(l) for l in res.stdout.splitlines() if l.startswith("{")], res.stderr


def test_sync_and_log_switches():
    base = {k: v for k, v in os.environ.items() if k not in ("QKV_PREP_LOG", "QKV_PREP_SYNC")}
    print("calls without the switches", flush=True)
    want, err_plain = run(base)
    print("calls with QKV_PREP_LOG=1 QKV_PREP_SYNC=1", flush=True)
    got, err = run(dict(base, QKV_PREP_LOG="1", QKV_PREP_SYNC="1"))
    assert len(want) == len(CALLS) and got == want
    assert "qkv_prep: launch shape" not in err_plain

    def key(s):
        return (s.rows_per_wave, s.kv_per_wave, s.waves_per_block, s.convert)

    cfg = qp.make_config(H)
    small, large = (key(qp.qkv_prep_launch_shape(cfg, 256, T)) for T in (16, 2048))
    assert small != large
    lines = [l for l in err.splitlines() if l.startswith("qkv_prep: launch shape")]
    shapes = [tuple(int(v) for v in re.findall(r"(?:rows/wave|kv/wave|waves/block|convert)=(\d+)", l))
              for l in lines]
    assert shapes == [small, large, small], err[-2000:]
