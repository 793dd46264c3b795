"""HIP path vs the CPU oracle, element by element, through the C ABI.

Every token of every case is compared (the oracle runs over token chunks on
the host cores); see tests/parity.py for the bar.  Inputs are drawn on the GPU
and copied to the host for the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_amd import workloads as W

from parity import CODE, EXP, assert_bit_exact, assert_within_bar, byte_roles, run_and_compare, tiny_weights

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(w, *, q_weight=True, exact=True, **cfg):
    note("case %s cfg=%s q_weight=%s" % (w.label, cfg, q_weight))
    inp = W.make_inputs(w, device=DEV, q_weight=True)
    res = run_and_compare(w, inp, q_weight=q_weight, **cfg)
    note("  -> %s" % res)
    if exact:
        assert_bit_exact(res)
    else:
        assert_within_bar(res)
    return res


# ----------------------------------------------------------------- workloads

@pytest.mark.parametrize("convert", [1, 2])
def test_tiny(convert):
    res = check(W.WORKLOADS["tiny"], convert=convert)
    assert res["valid_slots"] == 14


@pytest.mark.parametrize("convert", [1, 2])
def test_decode_2048x64(convert):
    check(W.WORKLOADS["decode"], convert=convert)


def test_prefill_32768x64():
    check(W.WORKLOADS["prefill"])


def test_prefill_wide_32768x128():
    check(W.WORKLOADS["prefill_wide"])


def test_long_131072x128():
    check(W.WORKLOADS["long"], exact=True)


# ----------------------------------------------------------------- launch shapes

SHAPES = [(1, 8), (4, 8), (17, 64), (64, 3), (511, 64), (777, 5), (1000, 1), (4096, 128)]


@pytest.mark.parametrize("T,H", SHAPES)
@pytest.mark.parametrize("rpw,wpb", [(u, b) for u in (1, 2, 4) for b in (1, 2, 4, 8)])
def test_forced_launch_shapes(T, H, rpw, wpb):
    check(W.custom(T, H, seed=100 + T + H), rows_per_wave=rpw, waves_per_block=wpb,
          convert=2 if (T + rpw) % 2 else 1)


@pytest.mark.parametrize("T,H", [(1, 48), (17, 96), (511, 48), (2049, 96), (4096, 48)])
def test_head_counts_the_pages_measure(T, H):
    # 48 and 96 heads appear in the pages' shape lists; default (heuristic)
    # launch, ragged token counts.
    check(W.custom(T, H, seed=300 + T + H, num_skip=min(3, T - 1)))
    check(W.custom(T, H, seed=301 + T + H), rows_per_wave=1)


@pytest.mark.parametrize("T,H", [(1, 8), (5, 3), (17, 64), (777, 5), (4099, 8)])
@pytest.mark.parametrize("kv_per_wave", [1, 2, 4])
def test_forced_kv_rows_per_wavefront(T, H, kv_per_wave):
    # 1, 2 or 4 consecutive tokens' kv rows per wavefront, at ragged token
    # counts (a last wavefront with fewer tokens), with skipped slots, under
    # both q shapes and both cache modes.
    w = W.custom(T, H, seed=340 + T + H, num_skip=min(T // 3, 7))
    for rpw in (1, 2):
        check(w, kv_per_wave=kv_per_wave, rows_per_wave=rpw)
    res = run_and_compare(w, W.make_inputs(w, device=DEV), kv_store=1, kv_per_wave=kv_per_wave)
    assert_bit_exact(res)


@pytest.mark.parametrize("T", [5, 777, 1001])
@pytest.mark.parametrize("kv_per_wave,wpb", [(2, 2), (4, 2), (4, 8), (2, 8)])
def test_kv_rows_per_wavefront_with_wider_workgroups(T, kv_per_wave, wpb):
    # Several kv wavefronts per workgroup, each taking several tokens: the
    # token index combines the workgroup, the wavefront and kv_per_wave.
    w = W.custom(T, 5, seed=350 + T + 10 * kv_per_wave + wpb, num_skip=min(T // 3, 7))
    for rpw in (1, 2):
        check(w, kv_per_wave=kv_per_wave, waves_per_block=wpb, rows_per_wave=rpw)


def _expected_shape(T, H):
    """The launch heuristic, restated: (q rows per wavefront, wavefronts per
    workgroup, kv tokens per wavefront)."""
    q = T * H
    if q >= 1 << 16:
        two = 1 < H <= 56 and T >= 1 << 14
        return (2, 2, 4) if two else (1, 1, 4)
    if q >= (3 << 13 if T > 8192 else 1 << 15 if T > 4096 else 3 << 14):
        return (1, 1, 4)
    if q >= 1 << 15 and T >= 2048:
        return (2, 2, 2)
    if T >= 3072 or (T >= 2048 and H % 2 == 1):
        return (1, 1, 2 if q >= 1 << 14 or T > 8192 else 1)
    return (2 if H > 1 else 1, 1, 1)


@pytest.mark.parametrize("T,H", [(1023, 64), (1024, 64), (511, 128), (512, 128), (8192, 8), (16384, 8),
                                 (16383, 16), (16384, 16), (2047, 16), (2048, 16), (4096, 8), (1024, 32),
                                 (4096, 12), (4096, 11), (4097, 8), (8193, 3), (8192, 3), (24576, 1),
                                 (3072, 2), (3071, 2), (2048, 7), (2047, 7), (2048, 11), (4096, 4),
                                 (4095, 4), (8193, 1), (8192, 1), (16384, 56), (16384, 57), (16383, 40)])
def test_both_sides_of_the_launch_thresholds(T, H):
    # Default launch on each side of each boundary of the heuristic: 2^16 q
    # rows; one row and four kv tokens from 49152, 2^15 (above 4096 tokens)
    # or 24576 (above 8192 tokens) q rows; the two-heads band from 2^15 q
    # rows and 2048 tokens; one row from 3072 tokens (2048 with an odd head
    # count); two kv tokens from 2^14 q rows or above 8192 tokens.
    from fp8_kv_cache_amd.qkv_prep import QkvPrep
    shape = QkvPrep(H).launch_shape(T)
    assert (shape.rows_per_wave, shape.waves_per_block, shape.kv_per_wave) == _expected_shape(T, H)
    check(W.custom(T, H, seed=330 + T + H, num_skip=5))


@pytest.mark.parametrize("T,H,cfg", [
    (29127, 9, {}), (29128, 9, {}), (131075, 2, {}), (65537, 5, {}), (40000, 16, {}),
    (29128, 9, {"kv_store": 1}), (50000, 7, {"waves_per_block": 1}), (60001, 12, {"waves_per_block": 4}),
    (8192, 64, {"rows_per_wave": 2, "kv_per_wave": 4}), (40000, 16, {"kv_per_wave": 2})])
def test_kv_workgroups_spread_through_the_grid(T, H, cfg):
    # Two heads and four kv tokens per wavefront from 2^18 q rows: the kv
    # workgroups sit every kv_period workgroups through the first 55-75% of
    # the grid instead of first.  Both sides of the threshold (29127 x 9 =
    # 2^18 - 1 rows), ragged and odd sizes, both cache modes, forced
    # workgroup widths and a forced two-heads shape at 64 heads; with two kv
    # tokens per wavefront the kv workgroups come first.
    from fp8_kv_cache_amd.qkv_prep import QkvPrep
    shape_cfg = {k: v for k, v in cfg.items() if k != "kv_store"}
    shape = QkvPrep(H, **shape_cfg).launch_shape(T)
    spread = shape.rows_per_wave == 2 and shape.kv_per_wave == 4 and T * H >= 1 << 18
    assert (shape.kv_period > 0) == spread
    check(W.custom(T, H, seed=360 + T + H, num_skip=7), **cfg)


def _random_cases(n, seed, few_heads=False):
    """n seeded configurations that mix every knob at once: ragged token and
    head counts (up to 2^18 q rows), block sizes, table lengths, skipped
    slots, outlier rows, eps, a weightless q, both cache modes, and every
    forced launch setting (0 = the heuristic).  With few_heads: 2048 to 65536
    tokens of 1 to 8 heads (the launch shapes that follow the token count),
    three cases in four at the heuristic's shape."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        if few_heads:
            T, H = int(rng.integers(2048, 65537)), int(rng.integers(1, 9))
        else:
            T = int(rng.integers(1, 4) if len(cases) < 3 else rng.integers(1, 6001))
            H = int(rng.integers(1, 161))
        if T * H > 1 << 18 and not few_heads:
            continue
        forced = not few_heads or rng.integers(4) == 0
        cases.append(dict(
            T=T, H=H, seed=int(rng.integers(1 << 30)),
            block_size=int(rng.choice([1, 3, 16, 64, 100, 256])),
            max_position=int(rng.choice([1, 7, 4096, 200000])),
            num_skip=int(rng.integers(0, min(T, 9) + 1)),
            outlier_frac=float(rng.choice([0.0, 0.01])),
            eps=float(rng.choice([0.0, 1e-6, 1e-2])),
            q_weight=bool(rng.integers(2)),
            kv_store=int(rng.integers(2)),
            rows_per_wave=int(rng.choice([0, 1, 2, 4])) if forced else 0,
            waves_per_block=int(rng.choice([0, 1, 2, 4, 8])) if forced else 0,
            kv_per_wave=int(rng.choice([0, 1, 2, 4])) if forced else 0,
            convert=int(rng.integers(3))))
    return cases


RANDOM_CASES = _random_cases(24, 20261202) + _random_cases(8, 20261203, few_heads=True)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=["%dx%d" % (c["T"], c["H"]) for c in RANDOM_CASES])
def test_seeded_random_configurations(case):
    c = dict(case)
    w = W.custom(c.pop("T"), c.pop("H"), seed=c.pop("seed"), max_position=c.pop("max_position"),
                 block_size=c.pop("block_size"), num_skip=c.pop("num_skip"),
                 outlier_frac=c.pop("outlier_frac"), eps=c.pop("eps"))
    note("case %s %s" % (w.label, case))
    inp = W.make_inputs(w, device=DEV)
    res = run_and_compare(w, inp, **c)
    note("  -> %s" % res)
    assert_bit_exact(res)


@pytest.mark.parametrize("rpw", [0, 1])
def test_exponent_clamp_and_subnormal_outputs(rpw):
    # Tiny weights: every kv block sits at the exponent clamp (scale byte 0)
    # with non-zero and subnormal codes, and many q outputs are subnormal bf16.
    w = W.custom(300, 4, seed=310)
    inp = W.make_inputs(w, device=DEV)
    inp["q_w"] = tiny_weights(311, -133, -115, DEV)
    inp["kv_w"] = tiny_weights(312, -133, -122, DEV)
    note("case tiny weights rows_per_wave=%d" % rpw)
    res = run_and_compare(w, inp, rows_per_wave=rpw)
    note("  -> %s" % res)
    assert_bit_exact(res)
    cache = inp["cache"].clone()
    from fp8_kv_cache_amd.qkv_prep import QkvPrep
    QkvPrep(4)(inp["q"].clone(), inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"],
               inp["slot_mapping"], cache)
    torch.cuda.synchronize()
    roles = byte_roles(inp["slot_mapping"].cpu().numpy(), w.num_blocks, w.block_size)
    flat = cache.cpu().numpy().reshape(-1)
    assert np.all(flat[roles == EXP] == 0)                      # every block at the clamp
    assert np.count_nonzero(flat[roles == CODE] & 0x7F) > 1000   # ... with real codes


def test_sum_of_squares_overflow():
    # Finite bf16 rows whose fp32 sum of squares overflows (x ~ 2^60..2^70):
    # inv = 1/sqrt(inf) = 0, so the row's outputs are +-0 (signs kept) and a
    # kv row becomes zero blocks (scale byte 0, codes +-0).
    w = W.custom(40, 4, seed=320)
    inp = W.make_inputs(w, device=DEV)
    inp["q"][3] *= 2.0 ** 70
    inp["q"][7, 1] *= 2.0 ** 60
    inp["kv"][5] *= 2.0 ** 70
    for rpw in (0, 1):
        note("case sum-of-squares overflow rows_per_wave=%d" % rpw)
        assert_bit_exact(run_and_compare(w, inp, rows_per_wave=rpw))


@pytest.mark.parametrize("T,H", [(1, 64), (17, 8), (512, 64), (2048, 128)])
def test_weightless_q(T, H):
    check(W.custom(T, H, seed=200 + T), q_weight=False)


@pytest.mark.parametrize("block_size", [1, 5, 16, 64, 256])
def test_block_sizes(block_size):
    check(W.custom(300, 8, seed=300 + block_size, block_size=block_size))


def test_skips_and_out_of_range_slots():
    w = W.custom(256, 16, seed=401, num_skip=40)
    inp = W.make_inputs(w, device=DEV)
    s = inp["slot_mapping"]
    cap = w.num_blocks * w.block_size
    s[3] = cap
    s[7] = cap + 12345
    s[9] = -(1 << 40)
    s[11] = 1 << 45
    res = run_and_compare(w, inp)
    note("skips -> %s" % res)
    assert_bit_exact(res)


def test_all_slots_skipped_and_empty_cache():
    w = W.custom(100, 8, seed=402, num_blocks=2, block_size=64)
    inp = W.make_inputs(w, device=DEV)
    inp["slot_mapping"].fill_(-1)
    res = run_and_compare(w, inp)
    assert res["valid_slots"] == 0
    assert_bit_exact(res)


def test_positions_at_both_ends_of_the_table():
    w = W.custom(64, 8, seed=403, max_position=77)
    inp = W.make_inputs(w, device=DEV)
    inp["positions"][::2] = 0
    inp["positions"][1::2] = 76
    assert_bit_exact(run_and_compare(w, inp))


@pytest.mark.parametrize("rpw", [1, 2])
def test_out_of_range_positions_are_clamped(rpw):
    # Positions outside [0, max_position) break a precondition; the kernel
    # clamps them into the table, so it reads only table rows, and those
    # tokens come out as if their position were clamped.  The clamped run is
    # checked against the oracle; the out-of-range run must equal it byte for
    # byte (every other token included).
    from fp8_kv_cache_amd.qkv_prep import QkvPrep
    w = W.custom(200, 8, seed=405, max_position=100, num_skip=3)
    inp = W.make_inputs(w, device=DEV)
    bad = inp["positions"].clone()
    for i, p in ((3, -1), (10, -2 ** 40), (20, 100), (30, 100 + 12345), (40, 2 ** 62)):
        bad[i] = p
    inp["positions"] = bad.clamp(0, 99)
    assert_bit_exact(run_and_compare(w, inp, rows_per_wave=rpw))
    op = QkvPrep(8, block_size=w.block_size, eps=w.eps, rows_per_wave=rpw)
    outs = []
    for pos in (inp["positions"], bad):
        q, cache = inp["q"].clone(), inp["cache"].clone()
        op(q, inp["kv"], inp["q_w"], inp["kv_w"], pos, inp["cos_sin"], inp["slot_mapping"], cache)
        outs.append((q, cache))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])


def test_outlier_rows_and_eps_zero():
    w = W.custom(512, 16, seed=404, outlier_frac=0.05, eps=0.0)
    assert_bit_exact(run_and_compare(w, W.make_inputs(w, device=DEV)))


# ----------------------------------------------------------------- hand case

def test_hand_derived_slot_on_gpu():
    # The kv slot whose every byte the oracle tests derive by hand: a row of
    # ones at eps = 0 and position 0 with crafted weights (zeros, -0, exact
    # 448, ties in E4M3, subnormal codes).
    from fp8_kv_cache_amd.qkv_prep import QkvPrep
    w = np.ones(512, np.float32)
    w[0] = 3.5
    w[64], w[65], w[66] = 3.5, 1.0625, 1.1875
    w[128:192] = -0.0
    w[192:256] = 448.0
    w[256:320] = 2.0 ** -10
    w[320], w[321], w[322] = 1.0, 2.0 ** -16, 3 * 2.0 ** -18
    w[323:384] = 2.0 ** -18
    w[384] = -3.5
    kvw = torch.from_numpy(oracle.f32_to_bf16(w).view(np.int16)).view(torch.bfloat16)
    for convert in (1, 2):
        nb, bs = 2, 4
        cache = torch.full((nb, bs * 584), 0xA5, dtype=torch.uint8, device=DEV)
        q = torch.ones((1, 1, 512), dtype=torch.bfloat16, device=DEV)
        kv = torch.ones((1, 512), dtype=torch.bfloat16, device=DEV)
        cs = torch.from_numpy(W.rope_table(8)).to(DEV)
        pos = torch.zeros(1, dtype=torch.int64, device=DEV)
        slot = torch.tensor([6], dtype=torch.int64, device=DEV)
        op = QkvPrep(1, block_size=bs, eps=0.0, convert=convert)
        op(q, kv, None, kvw.to(DEV), pos, cs, slot, cache)
        torch.cuda.synchronize()
        want = np.full((nb, bs * 584), 0xA5, np.uint8)
        q_want = oracle.qkv_prep(np.full((1, 1, 512), 0x3F80, np.uint16),
                                 np.full((1, 512), 0x3F80, np.uint16), None,
                                 oracle.f32_to_bf16(w), np.zeros(1, np.int64), W.rope_table(8),
                                 np.array([6]), want, nb, bs, 0.0)
        assert np.array_equal(cache.cpu().numpy(), want), convert
        assert np.array_equal(W.as_u16(q), q_want), convert


# ----------------------------------------------------------------- behaviour

def test_empty_batch_is_a_no_op():
    from fp8_kv_cache_amd.qkv_prep import QkvPrep
    w = W.custom(0, 8, seed=405)
    inp = W.make_inputs(w, device=DEV)
    before = inp["cache"].clone()
    op = QkvPrep(8)
    op(inp["q"], inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"],
       inp["slot_mapping"], inp["cache"])
    torch.cuda.synchronize()
    assert torch.equal(before, inp["cache"])


def test_repeat_runs_are_byte_identical():
    from fp8_kv_cache_amd.qkv_prep import QkvPrep
    w = W.custom(4096, 64, seed=406)
    inp = W.make_inputs(w, device=DEV)
    outs = []
    for _ in range(3):
        q = inp["q"].clone()
        c = inp["cache"].clone()
        QkvPrep(64)(q, inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"],
                    inp["slot_mapping"], c)
        torch.cuda.synchronize()
        outs.append((q.view(torch.int16).cpu(), c.cpu()))
    for q, c in outs[1:]:
        assert torch.equal(q, outs[0][0]) and torch.equal(c, outs[0][1])


def test_side_stream_and_conversion_modes_agree():
    from fp8_kv_cache_amd.qkv_prep import QkvPrep
    w = W.custom(1500, 32, seed=407)
    inp = W.make_inputs(w, device=DEV)
    results = []
    s = torch.cuda.Stream()
    for convert in (1, 2):
        q = inp["q"].clone()
        c = inp["cache"].clone()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            QkvPrep(32, convert=convert)(q, inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"],
                                         inp["cos_sin"], inp["slot_mapping"], c)
        s.synchronize()
        results.append((q.view(torch.int16).cpu(), c.cpu()))
    assert torch.equal(results[0][0], results[1][0])
    assert torch.equal(results[0][1], results[1][1])


def test_concurrent_streams_and_a_shared_handle():
    # The handle is read-only after create: two handles, and one handle used
    # on two streams at once, must give the serial results.
    from fp8_kv_cache_amd.qkv_prep import QkvPrep
    w1 = W.custom(3000, 16, seed=410, block_size=16)
    w2 = W.custom(2000, 48, seed=411)
    i1, i2 = W.make_inputs(w1, device=DEV), W.make_inputs(w2, device=DEV)
    op1, op2 = QkvPrep(16, block_size=16), QkvPrep(48)

    def run(op, inp, q, c):
        op(q, inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"], inp["slot_mapping"], c)

    ref = {}
    for key, op, inp in (("1", op1, i1), ("2", op2, i2)):
        q, c = inp["q"].clone(), inp["cache"].clone()
        run(op, inp, q, c)
        ref[key] = (q, c)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    jobs = [("1", op1, i1, s1), ("2", op2, i2, s2), ("1", op1, i1, s2), ("2", op2, i2, s1),
            ("1", op1, i1, s1), ("1", op1, i1, s2)]
    bufs = [(inp["q"].clone(), inp["cache"].clone()) for _, _, inp, _ in jobs]
    torch.cuda.synchronize()
    for (_, op, inp, s), (q, c) in zip(jobs, bufs):
        with torch.cuda.stream(s):
            run(op, inp, q, c)
    torch.cuda.synchronize()
    for (key, _, _, _), (q, c) in zip(jobs, bufs):
        assert torch.equal(q.view(torch.int16), ref[key][0].view(torch.int16))
        assert torch.equal(c, ref[key][1])


def test_bad_arguments_touch_nothing():
    from fp8_kv_cache_amd import qkv_prep as qp
    w = W.custom(64, 8, seed=408)
    inp = W.make_inputs(w, device=DEV)
    before_q = inp["q"].clone()
    before_c = inp["cache"].clone()
    op = qp.QkvPrep(8)
    args = qp.make_args(inp["q"], inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"],
                        inp["cos_sin"], inp["slot_mapping"], inp["cache"])
    args.q = args.q + 2                                   # misaligned
    with pytest.raises(qp.QkvPrepError) as e:
        qp.qkv_prep_run(op.handle, args, None)
    assert e.value.code == qp.ERR_MISALIGNED
    # a short kv tensor is stopped by the binding before it reaches the device
    with pytest.raises(ValueError):
        op(inp["q"], inp["kv"][:-1], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"],
           inp["slot_mapping"], inp["cache"])
    torch.cuda.synchronize()
    assert torch.equal(before_q, inp["q"]) and torch.equal(before_c, inp["cache"])


def test_probe_copy_copies():
    from fp8_kv_cache_amd import probe
    for n in (16, 4096 * 16 + 48, 3 << 20):
        src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=DEV)
        dst = torch.zeros_like(src)
        probe.qkv_prep_probe_copy(dst.data_ptr(), src.data_ptr(), n,
                               torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(src, dst)



def test_probe_update_increments_every_chunk_once():
    from fp8_kv_cache_amd import probe
    rng = np.random.default_rng(420)
    for n in (16, 64 * 16 + 48, 3 << 20):
        host = rng.integers(0, 2 ** 32, n // 4, dtype=np.uint64).astype(np.uint32)
        host[0:12:4] = 0xFFFFFFFF                             # wraps to 0
        buf = torch.from_numpy(host.view(np.int32).copy()).to(DEV)
        probe.qkv_prep_probe_update(buf.data_ptr(), n, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        got = buf.cpu().numpy().view(np.uint32).reshape(-1, 4)
        want = host.reshape(-1, 4).copy()
        want[:, 0] += np.uint32(1)
        assert np.array_equal(got, want)


# ----------------------------------------------------------------- readings R3 and R4

def _bf16_tensor(u16, shape):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16).reshape(shape)).view(torch.bfloat16).to(DEV)


def _one_row(x16, w16, eps, cs):
    """One token, one head: q row x16 with q weight w16, the same row and
    weight for kv, position 0 of the table cs, slot 0 of a poisoned
    one-block cache.  Returns (GPU q, GPU cache, oracle q, oracle cache)."""
    from fp8_kv_cache_amd.qkv_prep import QkvPrep
    q = _bf16_tensor(x16, (1, 1, 512))
    kv = _bf16_tensor(x16, (1, 512))
    w = _bf16_tensor(w16, (512,))
    pos = torch.zeros(1, dtype=torch.int64, device=DEV)
    slots = torch.zeros(1, dtype=torch.int64, device=DEV)
    table = torch.from_numpy(cs).to(DEV)
    cache = torch.full((1, 64 * 584), 0x5A, dtype=torch.uint8, device=DEV)
    want_cache = cache.cpu().numpy().copy()
    QkvPrep(1, block_size=64, eps=eps)(q, kv, w, w, pos, table, slots, cache)
    torch.cuda.synchronize()
    want_q = oracle.qkv_prep(x16.reshape(1, 1, 512), x16.reshape(1, 512), w16, w16, np.zeros(1, np.int64), cs,
                             np.zeros(1, np.int64), want_cache, 1, 64, eps)
    return W.as_u16(q), cache.cpu().numpy(), want_q, want_cache


def test_rows_where_the_readings_part_in_bf16():
    # The CPU pins fix the oracle to readings R3 (y = RN(RN(x*inv)*w)) and R4
    # (a' = RN(fma(a, c, -RN(b*s))), b' = RN(fma(a, s, RN(b*c)))) with cases
    # whose fp32 intermediates differ; these two rows are ones where the
    # alternatives also change a stored bf16 value, so the kernel's bits show
    # which reading it takes.
    from fractions import Fraction
    import mx_exact as X

    def bf16(v):
        return oracle.f32_to_bf16(np.asarray(v, np.float32))

    # R3: row 249 of seed 1000's normal rows, weights 1 + 0.1 N(0, 1), eps 1e-6,
    # the identity rotation: at dim 425, RN(RN(x*w)*inv) and RN(x*RN(inv*w))
    # both round to another bf16 than the stated order.
    rng = np.random.default_rng(1000)
    x = bf16(rng.standard_normal((256, 512)))[249]
    w = bf16(1.0 + 0.1 * rng.standard_normal(512))
    cs = W.rope_table(8)
    note("case R3 row (seed 1000, row 249)")
    got_q, got_cache, want_q, want_cache = _one_row(x, w, 1e-6, cs)
    assert np.array_equal(got_q.reshape(-1), want_q.reshape(-1))
    assert np.array_equal(got_cache, want_cache)
    _, _, _, inv = oracle.rows(x.reshape(1, 512), w, 1e-6, cs[:1])
    xf, wf, iv = (float(oracle.bf16_to_f32(x)[425]), float(oracle.bf16_to_f32(w)[425]), float(inv[0]))
    stated = X.rn32(Fraction(X.rn32(Fraction(xf) * Fraction(iv))) * Fraction(wf))
    others = (X.rn32(Fraction(X.rn32(Fraction(xf) * Fraction(wf))) * Fraction(iv)),
              X.rn32(Fraction(xf) * Fraction(X.rn32(Fraction(iv) * Fraction(wf)))))
    assert all(X.bf16(o) != X.bf16(stated) for o in others)
    assert got_q.reshape(-1)[425] == int(bf16([float(stated)])[0])

    # R4: a row of ones at eps = 0 (inv = 1, y = w) with the pairs set by the
    # weight; table row 0 is the identity except pairs 0 and 1, which take
    # float32 cos 7 and sin 7.  Pair 0 decides the first output, pair 1 the
    # second: both alternatives (two roundings; the fma on the other product)
    # give another bf16.
    c = float(np.uint32(0x3F40FFBD).view(np.float32))
    s = float(np.uint32(0x3F283046).view(np.float32))
    wv = np.ones(512, np.float32)
    wv[448:452] = (-0.90234375, -0.96875, -1.7734375, 1.4921875)
    w = bf16(wv)
    cs = np.zeros((8, 64), np.float32)
    cs[:, :32] = 1.0
    cs[0, 0] = cs[0, 1] = c
    cs[0, 32] = cs[0, 33] = s
    note("case R4 pairs at cos 7, sin 7")
    got_q, got_cache, want_q, want_cache = _one_row(bf16(np.ones(512)), w, 0.0, cs)
    assert np.array_equal(got_q.reshape(-1), want_q.reshape(-1))
    assert np.array_equal(got_cache, want_cache)
    C, S = Fraction(c), Fraction(s)
    a, b = Fraction(-0.90234375), Fraction(-0.96875)
    first = [X.rn32(a * C - X.rn32(b * S)), X.rn32(X.rn32(a * C) - X.rn32(b * S)), X.rn32(-b * S + X.rn32(a * C))]
    a, b = Fraction(-1.7734375), Fraction(1.4921875)
    second = [X.rn32(a * S + X.rn32(b * C)), X.rn32(X.rn32(a * S) + X.rn32(b * C)), X.rn32(b * C + X.rn32(a * S))]
    for vals, dim in ((first, 448), (second, 451)):
        assert X.bf16(vals[0]) != X.bf16(vals[1]) and X.bf16(vals[0]) != X.bf16(vals[2])
        assert got_q.reshape(-1)[dim] == int(bf16([float(vals[0])])[0])
