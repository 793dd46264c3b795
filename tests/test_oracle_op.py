"""Pins of the oracle's quantizer, cache insert and whole operator: a fully
hand-derived kv slot, dequantization error bounds, layout, skip rules and
untouched bytes, and the weight/identity closed forms end to end."""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_amd import workloads as W

SLOT = 584


def bf16(x):
    return oracle.f32_to_bf16(np.asarray(x, np.float32))


def run_oracle(inp, nthreads=1):
    cache = inp["cache"].numpy().copy()
    q_w = None if inp["q_w"] is None else W.as_u16(inp["q_w"])
    q_out = oracle.qkv_prep(W.as_u16(inp["q"]), W.as_u16(inp["kv"]), q_w,
                            W.as_u16(inp["kv_w"]), inp["positions"].numpy(),
                            inp["cos_sin"].numpy(), inp["slot_mapping"].numpy(), cache,
                            inp["num_blocks"], inp["block_size"], inp["eps"], nthreads)
    return q_out, cache


def dequant_slot(cache_flat, data_off, scale_off):
    d = cache_flat[data_off:data_off + 576]
    sc = cache_flat[scale_off:scale_off + 8]
    vals = oracle.e4m3_to_f64(d[:448]).reshape(7, 64) * np.ldexp(1.0, sc[:7].astype(int) - 127)[:, None]
    rope = oracle.bf16_to_f32(d[448:].view(np.uint16)).astype(np.float64)
    return vals.reshape(448), rope, sc


# ------------------------------------------------------------- hand-derived slot

def test_hand_derived_kv_slot():
    # kv row of ones at eps = 0 gives inv = 1 and y = w exactly; position 0 is
    # the identity rotation.  The weights are chosen per 64-block so that every
    # code and scale byte can be worked out by hand (see the golden codec file
    # for the format rules):
    w = np.ones(512, np.float32)
    w[0] = 3.5          # block 0: amax 3.5 -> e = -7 (byte 120); 3.5*2^7 = 448 -> 0x7e; 1*2^7 -> 0x70
    w[64] = 3.5         # block 1: amax 3.5, e = -7
    w[65] = 1.0625      #          1.0625*2^7 = 136, tie between 128 and 144 -> 0x70
    w[66] = 1.1875      #          152 = 1.1875*2^7, tie between 144 (m=1) and 160 (m=2) -> 0x72
    w[128:192] = -0.0   # block 2: all -0 -> amax 0 -> byte 0, codes 0x80
    w[192:256] = 448.0  # block 3: amax 448 -> e = 0 (byte 127); codes 0x7e
    w[256:320] = 2.0 ** -10   # block 4: e = -18 (byte 109); 2^-10*2^18 = 256 -> 0x78
    w[320] = 1.0        # block 5: amax 1 -> e = -8 (byte 119), 1*2^8 = 256 -> 0x78
    w[321] = 2.0 ** -16  #         2^-8 = 2*2^-9 -> 0x02
    w[322] = 3 * 2.0 ** -18   #   3*2^-10 = 1.5*2^-9, tie -> 2*2^-9 -> 0x02
    w[323] = 2.0 ** -18  #         2^-10 = 0.5*2^-9, tie -> 0 -> 0x00
    w[324:384] = 2.0 ** -18
    w[384] = -3.5       # block 6: amax 3.5, e = -7; -448 -> 0xfe, 1*2^7 -> 0x70
    # dims 448..511: w = 1 -> rope values 1.0 -> bf16 0x3f80
    exp_codes = np.zeros(448, np.uint8)
    exp_codes[0:64] = 0x70
    exp_codes[0] = 0x7E
    exp_codes[64:128] = 0x70
    exp_codes[64] = 0x7E
    exp_codes[65] = 0x70
    exp_codes[66] = 0x72
    exp_codes[128:192] = 0x80
    exp_codes[192:256] = 0x7E
    exp_codes[256:320] = 0x78
    exp_codes[320] = 0x78
    exp_codes[321] = 0x02
    exp_codes[322] = 0x02
    exp_codes[323:384] = 0x00
    exp_codes[384:448] = 0x70
    exp_codes[384] = 0xFE
    exp_scales = np.array([120, 120, 0, 127, 109, 119, 120, 0], np.uint8)

    nb, bs = 2, 4
    cache = np.full((nb, bs * SLOT), 0xA5, np.uint8)
    kv = bf16(np.ones((1, 512)))
    q = bf16(np.ones((1, 1, 512)))
    cs = W.rope_table(8)
    slot = 6                                      # block 1, slot 2
    q_out = oracle.qkv_prep(q, kv, None, bf16(w), np.array([0]), cs, np.array([slot]),
                            cache, nb, bs, 0.0)
    flat = cache.reshape(-1)
    data_off = 1 * bs * SLOT + 2 * 576
    scale_off = 1 * bs * SLOT + bs * 576 + 2 * 8
    assert oracle.slot_offsets(slot, nb, bs) == (data_off, scale_off)
    assert np.array_equal(flat[data_off:data_off + 448], exp_codes)
    assert np.array_equal(flat[data_off + 448:data_off + 576].view(np.uint16),
                          np.full(64, 0x3F80, np.uint16))
    assert np.array_equal(flat[scale_off:scale_off + 8], exp_scales)
    # everything else untouched
    mask = np.ones(flat.size, bool)
    mask[data_off:data_off + 576] = False
    mask[scale_off:scale_off + 8] = False
    assert np.all(flat[mask] == 0xA5)
    # weightless q of ones at position 0 comes back as ones
    assert np.all(q_out == 0x3F80)


# ------------------------------------------------------------- bounds

def test_dequantized_kv_within_e4m3_bound():
    w = W.custom(256, 4, seed=21)
    inp = W.make_inputs(w)
    _, cache = run_oracle(inp)
    flat = cache.reshape(-1)
    x = W.as_u16(inp["kv"])
    cs = inp["cos_sin"].numpy()[inp["positions"].numpy()]
    y, z, _, _ = oracle.rows(x, W.as_u16(inp["kv_w"]), inp["eps"], cs)
    for t, slot in enumerate(inp["slot_mapping"].numpy()):
        d_off, s_off = oracle.slot_offsets(slot, w.num_blocks, w.block_size)
        vals, rope, sc = dequant_slot(flat, d_off, s_off)
        e = sc[:7].astype(int) - 127
        step = np.repeat(np.ldexp(1.0, e - 9), 64)         # subnormal spacing per block
        yt = y[t, :448].astype(np.float64)
        # round to nearest with 3 mantissa bits: half-step 2^-4 relative, or half
        # the subnormal step in absolute terms
        assert np.all(np.abs(vals - yt) <= np.maximum(2.0 ** -4 * np.abs(yt), step / 2))
        # every scaled value fits 448, and the exponent is the least that does
        amax = np.abs(yt).reshape(7, 64).max(axis=1)
        assert np.all(amax <= 448.0 * np.ldexp(1.0, e))
        assert np.all(amax > 448.0 * np.ldexp(1.0, e - 1))
        # rope dims are the bf16 of the rotated fp32 values
        assert np.array_equal(bf16(z[t, 448:]), flat[d_off + 448:d_off + 576].view(np.uint16))
        assert sc[7] == 0


def test_skipped_and_out_of_range_slots_write_nothing():
    w = W.custom(40, 8, seed=22, num_blocks=2, block_size=32)   # 64 slots
    inp = W.make_inputs(w)
    slots = inp["slot_mapping"].clone()
    slots[3] = -1
    slots[5] = -7
    slots[9] = 64          # == capacity
    slots[11] = 1 << 40
    inp["slot_mapping"] = slots
    before = inp["cache"].numpy().copy()
    _, cache = run_oracle(inp)
    valid = [s for s in slots.tolist() if 0 <= s < 64]
    touched = np.zeros(before.size, bool)
    for s in valid:
        d, sc = oracle.slot_offsets(s, 2, 32)
        touched[d:d + 576] = True
        touched[sc:sc + 8] = True
    assert np.array_equal(cache.reshape(-1)[~touched], before.reshape(-1)[~touched])
    assert len(valid) == 36


def test_whole_op_q_matches_rows_and_threads_agree():
    w = W.WORKLOADS["tiny"]
    inp = W.make_inputs(w)
    q_out, cache = run_oracle(inp)
    q_out4, cache4 = run_oracle(inp, nthreads=4)
    assert np.array_equal(q_out, q_out4) and np.array_equal(cache, cache4)
    x = W.as_u16(inp["q"]).reshape(-1, 512)
    cs = np.repeat(inp["cos_sin"].numpy()[inp["positions"].numpy()], w.num_heads, axis=0)
    _, z, _, _ = oracle.rows(x, W.as_u16(inp["q_w"]), inp["eps"], cs)
    assert np.array_equal(q_out.reshape(-1, 512), bf16(z))
    # exactly 14 of 16 tokens have a slot
    assert int((inp["slot_mapping"] >= 0).sum()) == 14


def test_preallocated_output_gives_the_same_result():
    w = W.WORKLOADS["tiny"]
    inp = W.make_inputs(w)
    q_out, cache = run_oracle(inp)
    out = np.full_like(q_out, 0xFFFF)
    cache2 = inp["cache"].numpy().copy()
    got = oracle.qkv_prep(W.as_u16(inp["q"]), W.as_u16(inp["kv"]), W.as_u16(inp["q_w"]),
                          W.as_u16(inp["kv_w"]), inp["positions"].numpy(), inp["cos_sin"].numpy(),
                          inp["slot_mapping"].numpy(), cache2, inp["num_blocks"], inp["block_size"],
                          inp["eps"], 2, out=out)
    assert got is out and np.array_equal(out, q_out) and np.array_equal(cache2, cache)
    with pytest.raises(TypeError):
        oracle.qkv_prep(W.as_u16(inp["q"]), W.as_u16(inp["kv"]), None, W.as_u16(inp["kv_w"]),
                        inp["positions"].numpy(), inp["cos_sin"].numpy(), inp["slot_mapping"].numpy(),
                        cache2, inp["num_blocks"], inp["block_size"], inp["eps"], 1, out=out[:1])


def test_whole_op_q_against_float64_ideal():
    # bf16 output of the fp32 chain vs the float64 evaluation of the same
    # formula: at most one bf16 ulp apart (the fp32 error is ~2^-20 relative,
    # far below bf16's 2^-8, so only values near a rounding tie can differ).
    w = W.custom(64, 8, seed=23, max_position=131072)
    inp = W.make_inputs(w)
    q_out, _ = run_oracle(inp)
    xf = oracle.bf16_to_f32(W.as_u16(inp["q"])).astype(np.float64)
    wf = oracle.bf16_to_f32(W.as_u16(inp["q_w"])).astype(np.float64)
    cs = inp["cos_sin"].numpy()[inp["positions"].numpy()].astype(np.float64)
    inv = 1.0 / np.sqrt((xf ** 2).mean(axis=-1, keepdims=True) + np.float64(np.float32(1e-6)))
    y = xf * inv * wf
    a, b = y[..., 448::2].copy(), y[..., 449::2].copy()
    c, s = cs[:, None, :32], cs[:, None, 32:]
    y[..., 448::2] = a * c - b * s
    y[..., 449::2] = a * s + b * c
    got = oracle.bf16_to_f32(q_out).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(y))[1] - 8)
    assert np.all(np.abs(got - y) <= ulp)


def test_eps_zero_constant_rows_give_weights_at_position_zero():
    T, H = 3, 4
    q = bf16(np.ones((T, H, 512)))
    kv = bf16(np.ones((T, 512)))
    rng = np.random.default_rng(30)
    q_w = bf16(1 + 0.1 * rng.standard_normal(512))
    cache = np.zeros((1, 64 * SLOT), np.uint8)
    out = oracle.qkv_prep(q, kv, q_w, bf16(np.ones(512)), np.zeros(T, np.int64),
                          W.rope_table(4), np.array([0, 1, 2]), cache, 1, 64, 0.0)
    assert np.all(out == q_w[None, None, :])


def test_bad_position_is_rejected_and_writes_nothing():
    cache = np.zeros((1, 64 * SLOT), np.uint8)
    with pytest.raises(ValueError):
        oracle.qkv_prep(bf16(np.ones((1, 1, 512))), bf16(np.ones((1, 512))), None,
                        bf16(np.ones(512)), np.array([4]), W.rope_table(4),
                        np.array([0]), cache, 1, 64, 1e-6)
    assert not cache.any()
