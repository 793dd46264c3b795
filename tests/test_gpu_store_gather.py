"""GPU checks of the bf16-store cache mode and of the cache reader, through
the C ABI, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_amd import qkv_prep as qp
from fp8_kv_cache_amd import workloads as W

from parity import assert_bit_exact, run_and_compare, tiny_weights

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def note(msg):
    print(msg, flush=True)


# ----------------------------------------------------------------- bf16 store

@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_bf16_store_workloads(name):
    w = W.WORKLOADS[name]
    note("bf16 store %s" % w.label)
    res = run_and_compare(w, W.make_inputs(w, device=DEV), kv_store=qp.KV_BF16)
    note("  -> %s" % res)
    assert_bit_exact(res)


@pytest.mark.parametrize("T,H,bs,convert", [(1, 8, 1, 1), (17, 3, 5, 2), (777, 64, 16, 1),
                                            (2048, 128, 64, 2)])
def test_bf16_store_shapes(T, H, bs, convert):
    w = W.custom(T, H, seed=600 + T, block_size=bs, num_skip=min(T // 4, 10))
    res = run_and_compare(w, W.make_inputs(w, device=DEV), kv_store=qp.KV_BF16, convert=convert)
    assert_bit_exact(res)


# ----------------------------------------------------------------- reader

def _insert(w, inp):
    op = qp.QkvPrep(w.num_heads, block_size=w.block_size, eps=w.eps)
    q = inp["q"].clone()
    cache = inp["cache"].clone()
    op(q, inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"],
       inp["slot_mapping"], cache)
    torch.cuda.synchronize()
    return op, cache


@pytest.mark.parametrize("name,bs", [("decode", None), ("custom", 5), ("custom", 1)])
def test_gather_matches_the_oracle_reader(name, bs):
    w = W.WORKLOADS["decode"] if name == "decode" else W.custom(500, 4, seed=700 + bs,
                                                                 block_size=bs, num_skip=9)
    inp = W.make_inputs(w, device=DEV)
    op, cache = _insert(w, inp)
    cap = w.num_blocks * w.block_size
    slots = inp["slot_mapping"].clone()
    extra = torch.tensor([-1, cap, cap + 7, -(1 << 40), 1 << 40], dtype=torch.int64, device=DEV)
    probe = torch.cat([slots.flip(0), extra])              # out of order, plus invalid slots
    host_cache = cache.cpu().numpy()
    want = oracle.gather_dequant(host_cache, w.num_blocks, w.block_size, probe.cpu().numpy())
    out32 = torch.full((probe.numel(), 512), float("nan"), dtype=torch.float32, device=DEV)
    op.gather(cache, probe, out32)
    out16 = torch.full((probe.numel(), 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    op.gather(cache, probe, out16)
    torch.cuda.synchronize()
    got32 = out32.cpu().numpy()
    assert np.array_equal(got32.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(W.as_u16(out16), oracle.f32_to_bf16(want))
    assert np.all(got32[-len(extra):] == 0)


def test_gather_round_trip_within_e4m3_bound():
    w = W.custom(1024, 8, seed=710)
    inp = W.make_inputs(w, device=DEV)
    op, cache = _insert(w, inp)
    out = torch.empty((w.num_tokens, 512), dtype=torch.float32, device=DEV)
    op.gather(cache, inp["slot_mapping"], out)
    torch.cuda.synchronize()
    cs = inp["cos_sin"].cpu().numpy()[inp["positions"].cpu().numpy()]
    y, z, _, _ = oracle.rows(W.as_u16(inp["kv"]), W.as_u16(inp["kv_w"]), w.eps, cs)
    got = out.cpu().numpy().astype(np.float64)
    _, scales = oracle.quant_rows(y[:, :448])
    e = np.repeat(scales.astype(int) - 127, 64, axis=1)
    assert np.all(np.abs(got[:, :448] - y[:, :448]) <=
                  np.maximum(2.0 ** -4 * np.abs(y[:, :448]), np.ldexp(1.0, e - 10)))
    assert np.array_equal(out.cpu().numpy()[:, 448:], oracle.bf16_to_f32(oracle.f32_to_bf16(z[:, 448:])))


def test_gather_empty_and_bad_arguments():
    w = W.custom(64, 8, seed=711)
    inp = W.make_inputs(w, device=DEV)
    op, cache = _insert(w, inp)
    out = torch.zeros((0, 512), dtype=torch.float32, device=DEV)
    op.gather(cache, inp["slot_mapping"][:0], out)          # n == 0: no-op
    out = torch.zeros((4, 512), dtype=torch.float32, device=DEV)
    args = qp.QkvPrepGatherArgs(cache.data_ptr(), w.num_blocks, inp["slot_mapping"].data_ptr(), 4,
                                out.data_ptr() + 4, qp.OUT_F32)
    with pytest.raises(qp.QkvPrepError) as e:
        qp.qkv_prep_gather(op.handle, args, None)
    assert e.value.code == qp.ERR_MISALIGNED
    args = qp.QkvPrepGatherArgs(cache.data_ptr(), w.num_blocks, inp["slot_mapping"].data_ptr(), 4,
                                out.data_ptr(), 7)
    with pytest.raises(qp.QkvPrepError) as e:
        qp.qkv_prep_gather(op.handle, args, None)
    assert e.value.code == qp.ERR_INVALID_ARG
    bf = qp.QkvPrep(8, kv_store=qp.KV_BF16)
    args = qp.QkvPrepGatherArgs(cache.data_ptr(), w.num_blocks, inp["slot_mapping"].data_ptr(), 4,
                                out.data_ptr(), qp.OUT_F32)
    with pytest.raises(qp.QkvPrepError) as e:
        qp.qkv_prep_gather(bf.handle, args, None)
    assert e.value.code == qp.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == 0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gather_from_an_empty_cache_reads_zero_rows(dtype):
    # num_blocks 0 and no cache at all: every slot is out of range, so every
    # row reads as zeros and the (absent) cache is never touched.
    slots = torch.tensor([0, 1, -1, 5, 100, 2 ** 40], dtype=torch.int64, device=DEV)
    out = torch.full((slots.numel(), 512), 7.0, dtype=dtype, device=DEV)
    op = qp.QkvPrep(8, block_size=64)
    args = qp.QkvPrepGatherArgs(None, 0, slots.data_ptr(), slots.numel(), out.data_ptr(),
                                qp.OUT_F32 if dtype == torch.float32 else qp.OUT_BF16)
    qp.qkv_prep_gather(op.handle, args, None)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and not torch.any(torch.signbit(out))


def _nan_aware_equal(got_bits, want_bits, nan_mask_got, nan_mask_want):
    """Equal bit patterns, except that a NaN may carry any payload."""
    return np.array_equal(nan_mask_got, nan_mask_want) and \
        np.array_equal(got_bits[~nan_mask_want], want_bits[~nan_mask_want])


@pytest.mark.parametrize("bs,nb", [(64, 96), (7, 300)])
def test_gather_arbitrary_cache_bytes(bs, nb):
    # Every byte of the cache random: all 256 codes (NaN codes 0x7f/0xff
    # included), every scale byte 0..255 and random rope bf16.  Every slot is
    # read once in a random order, plus invalid slots.  Byte 255 (scale 2^128)
    # is also forced on some blocks whose codes include 0x00 and 0x80, which
    # must read back as +0 and -0.
    note("gather arbitrary bytes: block_size %d, %d blocks" % (bs, nb))
    rng = np.random.default_rng(720 + bs)
    host = rng.integers(0, 256, (nb, bs * W.SLOT_BYTES), dtype=np.uint8)
    rec = host[:, bs * 576:].reshape(nb, bs, 8)
    rec[::5, :, 0] = 255
    data = host[:, : bs * 576].reshape(nb, bs, 576)
    data[::5, :, 0] = 0x00
    data[::5, :, 1] = 0x80
    cap = nb * bs
    probe = np.concatenate([rng.permutation(cap), [-1, cap, -5, cap + 1]]).astype(np.int64)
    want = oracle.gather_dequant(host, nb, bs, probe)
    cache = torch.from_numpy(host).to(DEV)
    slots = torch.from_numpy(probe).to(DEV)
    op = qp.QkvPrep(8, block_size=bs)
    out32 = torch.full((probe.size, 512), 7.0, dtype=torch.float32, device=DEV)
    out16 = torch.full((probe.size, 512), 7.0, dtype=torch.bfloat16, device=DEV)
    op.gather(cache, slots, out32)
    op.gather(cache, slots, out16)
    torch.cuda.synchronize()
    got32 = out32.cpu().numpy()
    assert np.isnan(want).any() and np.isinf(want).any()        # the odd values are exercised
    cases = np.arange(cap)[np.argsort(probe[:cap])]             # row of each slot
    zero_rows = cases.reshape(nb, bs)[::5].reshape(-1)
    assert np.all(want[zero_rows, 0] == 0) and not np.signbit(want[zero_rows, 0]).any()
    assert np.all(want[zero_rows, 1] == 0) and np.signbit(want[zero_rows, 1]).all()
    assert _nan_aware_equal(got32.view(np.uint32), want.view(np.uint32), np.isnan(got32), np.isnan(want))
    got16 = W.as_u16(out16)
    want16 = oracle.f32_to_bf16(want)
    is_nan16 = lambda u: ((u & 0x7F80) == 0x7F80) & ((u & 0x007F) != 0)
    assert _nan_aware_equal(got16, want16, is_nan16(got16), np.isnan(want))
    assert np.all(got32[cap:] == 0) and np.all(got16[cap:] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gather_full_cache_block_walk(dtype):
    # The benchmarked configuration: every slot of the 4096 x 64-slot cache as
    # a block-table walk (blocks shuffled, slots in order), here with the last
    # 3 rows dropped so that the final window of rows is ragged.
    w = W.WORKLOADS["decode"]
    bs, nb = w.block_size, w.num_blocks
    note("gather full cache %s: %d x %d slots" % (dtype, nb, bs))
    rng = np.random.default_rng(730)
    host = rng.integers(0, 256, (nb, bs * W.SLOT_BYTES), dtype=np.uint8)
    host[:, bs * 576:] = rng.integers(100, 140, (nb, bs * 8), dtype=np.uint8)
    probe = (rng.permutation(nb)[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)[:-3].astype(np.int64)
    want = oracle.gather_dequant(host, nb, bs, probe)
    cache = torch.from_numpy(host).to(DEV)
    op = qp.QkvPrep(w.num_heads, block_size=bs)
    out = torch.full((probe.size, 512), 7.0, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                     device=DEV)
    op.gather(cache, torch.from_numpy(probe).to(DEV), out)
    torch.cuda.synchronize()
    if dtype == "f32":
        got = out.cpu().numpy()
        assert _nan_aware_equal(got.view(np.uint32), want.view(np.uint32), np.isnan(got), np.isnan(want))
    else:
        got = W.as_u16(out)
        is_nan16 = ((got & 0x7F80) == 0x7F80) & ((got & 0x007F) != 0)
        assert _nan_aware_equal(got, oracle.f32_to_bf16(want), is_nan16, np.isnan(want))


def test_subnormal_values_in_the_bf16_store_and_the_reader():
    # Tiny weights: the bf16-store slots hold subnormal bf16 values, and the
    # FP8 slots sit at the exponent clamp (scale 2^-127), so the reader's
    # products code * 2^-127 are fp32 subnormals.
    w = W.custom(300, 4, seed=740)
    inp = W.make_inputs(w, device=DEV)
    inp["q_w"] = tiny_weights(741, -133, -115, DEV)
    inp["kv_w"] = tiny_weights(742, -133, -122, DEV)
    note("tiny weights: bf16 store")
    assert_bit_exact(run_and_compare(w, inp, kv_store=qp.KV_BF16))
    note("tiny weights: reader")
    op, cache = _insert(w, inp)
    slots = inp["slot_mapping"]
    want = oracle.gather_dequant(cache.cpu().numpy(), w.num_blocks, w.block_size, slots.cpu().numpy())
    out32 = torch.empty((slots.numel(), 512), dtype=torch.float32, device=DEV)
    out16 = torch.empty((slots.numel(), 512), dtype=torch.bfloat16, device=DEV)
    op.gather(cache, slots, out32)
    op.gather(cache, slots, out16)
    torch.cuda.synchronize()
    got = out32.cpu().numpy()
    sub = (np.abs(want) < np.float32(2.0 ** -126)) & (want != 0)
    assert np.count_nonzero(sub) > 1000                      # fp32 subnormals really occur
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(W.as_u16(out16), oracle.f32_to_bf16(want))
