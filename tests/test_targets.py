"""Byte counts of the measured targets (host only): each target's algorithmic
bytes agree with the per-workload formulas and with the library's own size
function."""
import pytest

from fp8_kv_cache_amd import variants as V
from fp8_kv_cache_amd import workloads as W


def test_operator_targets_match_the_workload_formula():
    for name, w in W.WORKLOADS.items():
        t = V.target(name)
        assert t.alg_bytes == W.algorithmic_bytes(w.num_tokens, w.num_heads, w.num_tokens - w.num_skip)
    # hand figures: 2048 H + 1296 + 584 per token, plus 2 KiB of weights
    assert V.target("tiny").alg_bytes == 16 * (2048 * 8 + 1296) + 584 * 14 + 2048 == 293104
    assert V.target("prefill").alg_bytes == 4356573184
    assert V.target("long").alg_bytes == 34606155776


def test_variant_targets():
    t = V.target("bf16store_prefill")
    assert t.alg_bytes == W.algorithmic_bytes(32768, 64, 32768, slot_bytes=1024)
    for name, per in (("gather_bf16", 2), ("gather_f32", 4), ("gather_f32_shuffled", 4)):
        t = V.target(name)
        assert t.alg_bytes == W.gather_bytes(262144, 262144, per)
    t = V.target("mxfp8")
    m, h = 16384, 7168
    assert t.read_bytes == 4 * m * h + 2 * h
    assert t.write_bytes == 3 * m * h + 128 * 224 * 128        # 128 row tiles of 128 x 224 scales
    with pytest.raises(KeyError):
        V.target("nope")


def test_scale_size_matches_the_library():
    qp = pytest.importorskip("fp8_kv_cache_amd.qkv_prep")
    for m, h in ((1, 512), (130, 1536), (16384, 7168), (1000, 8192), (129, 4096)):
        assert V.mxfp8_scale_bytes(m, h) == qp.qkv_prep_mxfp8_scale_bytes(m, h)
