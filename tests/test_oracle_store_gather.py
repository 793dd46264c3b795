"""Pins of the oracle's bf16-store variant and of its cache reader
(dequantize-and-gather): closed forms from the per-row intermediates (pinned in
test_oracle_row.py), a hand-derived slot read back value by value, skip rules
and the E4M3 round-trip bound."""
import numpy as np

import oracle
from fp8_kv_cache_amd import workloads as W


def bf16(x):
    return oracle.f32_to_bf16(np.asarray(x, np.float32))


# ------------------------------------------------------------- bf16 store

def test_bf16_store_slot_is_the_bf16_of_the_rotated_row():
    w = W.custom(200, 4, seed=51, num_skip=20)
    inp = W.make_inputs(w)
    cache = np.full((w.num_blocks, w.block_size * 1024), 0x5A, np.uint8)
    q_out = oracle.qkv_prep(W.as_u16(inp["q"]), W.as_u16(inp["kv"]), W.as_u16(inp["q_w"]),
                            W.as_u16(inp["kv_w"]), inp["positions"].numpy(),
                            inp["cos_sin"].numpy(), inp["slot_mapping"].numpy(), cache,
                            w.num_blocks, w.block_size, w.eps, kv_store="bf16")
    cs = inp["cos_sin"].numpy()[inp["positions"].numpy()]
    _, z, _, _ = oracle.rows(W.as_u16(inp["kv"]), W.as_u16(inp["kv_w"]), w.eps, cs)
    flat = cache.reshape(-1)
    written = np.zeros(flat.size, bool)
    for t, s in enumerate(inp["slot_mapping"].numpy()):
        if s < 0:
            continue
        got = flat[s * 1024:(s + 1) * 1024].view(np.uint16)
        assert np.array_equal(got, bf16(z[t]))
        written[s * 1024:(s + 1) * 1024] = True
    assert np.all(flat[~written] == 0x5A)
    assert written.sum() == 180 * 1024
    # q is the same as with the FP8 cache
    cache8 = inp["cache"].numpy().copy()
    q8 = oracle.qkv_prep(W.as_u16(inp["q"]), W.as_u16(inp["kv"]), W.as_u16(inp["q_w"]),
                         W.as_u16(inp["kv_w"]), inp["positions"].numpy(), inp["cos_sin"].numpy(),
                         inp["slot_mapping"].numpy(), cache8, w.num_blocks, w.block_size, w.eps)
    assert np.array_equal(q_out, q8)


def test_bf16_store_constant_row_stores_the_weight():
    rng = np.random.default_rng(52)
    kv_w = bf16(1 + 0.1 * rng.standard_normal(512))
    cache = np.zeros((1, 8 * 1024), np.uint8)
    oracle.qkv_prep(bf16(np.ones((1, 1, 512))), bf16(np.ones((1, 512))), None, kv_w,
                    np.array([0]), W.rope_table(2), np.array([5]), cache, 1, 8, 0.0,
                    kv_store="bf16")
    assert np.array_equal(cache.reshape(-1)[5 * 1024:6 * 1024].view(np.uint16), kv_w)


# ------------------------------------------------------------- gather

def _hand_slot_cache():
    # The hand-derived slot of test_oracle_op.test_hand_derived_kv_slot.
    w = np.ones(512, np.float32)
    w[0] = 3.5
    w[64], w[65], w[66] = 3.5, 1.0625, 1.1875
    w[128:192] = -0.0
    w[192:256] = 448.0
    w[256:320] = 2.0 ** -10
    w[320], w[321], w[322] = 1.0, 2.0 ** -16, 3 * 2.0 ** -18
    w[323:384] = 2.0 ** -18
    w[384] = -3.5
    nb, bs = 2, 4
    cache = np.full((nb, bs * 584), 0xA5, np.uint8)
    oracle.qkv_prep(bf16(np.ones((1, 1, 512))), bf16(np.ones((1, 512))), None, bf16(w),
                    np.array([0]), W.rope_table(8), np.array([6]), cache, nb, bs, 0.0)
    return w, cache, nb, bs


def test_gather_reads_the_hand_derived_slot_back():
    w, cache, nb, bs = _hand_slot_cache()
    out = oracle.gather_dequant(cache, nb, bs, np.array([6]))[0]
    want = w.copy()
    want[65] = 1.0                 # 136 * 2^-7 rounded to 128 * 2^-7
    want[66] = 1.25                # 152 * 2^-7 rounded to 160 * 2^-7
    want[322] = 2.0 ** -16         # 1.5 * 2^-9 * 2^8 rounded to 2 * 2^-9 * 2^8
    want[323:384] = 0.0            # 0.5 * 2^-9 (scaled) rounded to 0
    assert np.array_equal(out, want)
    assert np.all(np.signbit(out[128:192]))        # -0 codes read back as -0
    assert np.array_equal(out[448:], np.ones(64, np.float32))


def test_gather_of_skipped_slots_is_zero_and_of_valid_slots_matches_rows():
    w = W.custom(300, 2, seed=53, block_size=16)
    inp = W.make_inputs(w)
    cache = inp["cache"].numpy().copy()
    oracle.qkv_prep(W.as_u16(inp["q"]), W.as_u16(inp["kv"]), W.as_u16(inp["q_w"]),
                    W.as_u16(inp["kv_w"]), inp["positions"].numpy(), inp["cos_sin"].numpy(),
                    inp["slot_mapping"].numpy(), cache, w.num_blocks, w.block_size, w.eps)
    slots = inp["slot_mapping"].numpy()
    probe = np.concatenate([slots, [-1, w.num_blocks * w.block_size, 1 << 40]])
    out = oracle.gather_dequant(cache, w.num_blocks, w.block_size, probe)
    assert np.all(out[len(slots):] == 0)
    cs = inp["cos_sin"].numpy()[inp["positions"].numpy()]
    y, z, _, _ = oracle.rows(W.as_u16(inp["kv"]), W.as_u16(inp["kv_w"]), w.eps, cs)
    got = out[:len(slots)].astype(np.float64)
    # rope dims: exactly the bf16 of the rotated values
    assert np.array_equal(out[:len(slots), 448:], oracle.bf16_to_f32(bf16(z[:, 448:])))
    # nope dims: within the E4M3 round-to-nearest bound of y
    codes, scales = oracle.quant_rows(y[:, :448])
    e = np.repeat(scales.astype(int) - 127, 64, axis=1)
    bound = np.maximum(2.0 ** -4 * np.abs(y[:, :448]), np.ldexp(1.0, e - 10))
    assert np.all(np.abs(got[:, :448] - y[:, :448]) <= bound)
    # and exactly code * 2^e of the oracle's own quantizer
    want = oracle.e4m3_to_f64(codes) * np.ldexp(1.0, e)
    assert np.array_equal(got[:, :448], want)
