"""The largest batches one MI355X holds.  From about 2^26 q rows the
operator's grid passes the 2^32 work-items one dispatch takes, so it is
enqueued as consecutive dispatches of the same kernel (two at 600000 x 128,
three at 1100000 x 128, two at 2400000 x 56 with two heads per wavefront and
the kv workgroups spread), each starting at its own workgroup index.  q
alone is 79, 144 and 138 GB here.  Every token cannot be
checked on the host at this size, so a seeded sample of tokens (the first, the
last, skipped ones and random ones) is checked one by one against the oracle:
each sampled token's q rows bit for bit, and its cache slot byte for byte (the
oracle writes the token into a one-block cache at the same offset within the
block, which is laid out like any other block)."""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_amd import qkv_prep as qp
from fp8_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SAMPLE = 48


def note(msg):
    print(msg, flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T,H,dispatches", [(600000, 128, 2), (1100000, 128, 3), (2400000, 56, 2)])
def test_largest_batches_on_sampled_tokens(T, H, dispatches):
    # 2400000 x 56: two heads per wavefront, two wavefronts per workgroup,
    # and the kv workgroups spread through the grid, over two dispatches.
    w = W.custom(T, H, seed=T // 1000 + H, num_skip=7)
    need = T * H * 1024 + T * 1024 + w.num_blocks * w.block_size * qp.SLOT_BYTES + (2 << 30)
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if need > free:
        pytest.skip("needs %.0f GB of free device memory, %.0f GB free" % (need / 1e9, free / 1e9))
    op = qp.QkvPrep(H, block_size=w.block_size, eps=w.eps)
    shape = op.launch_shape(T)
    if H > 56:
        assert shape.rows_per_wave == 1 and shape.waves_per_block == 1 and shape.kv_period == 0
    else:
        assert shape.rows_per_wave == 2 and shape.waves_per_block == 2 and shape.kv_period > 0
    per = (2 ** 32 - 1) // (64 * shape.waves_per_block)     # workgroups one dispatch takes
    assert -(-shape.grid // per) == dispatches
    note("case %s: drawing inputs (q %.0f GB), launch %s" % (
        w.label, T * H * 1024 / 1e9, (shape.rows_per_wave, shape.kv_per_wave, shape.grid, shape.kv_period)))
    inp = W.make_inputs(w, device=DEV)
    try:
        slots_all = inp["slot_mapping"]
        skipped = torch.nonzero(slots_all < 0).flatten()
        rng = np.random.default_rng(T)
        picks = set(rng.choice(T, SAMPLE, replace=False).tolist()) | {0, T - 1}
        picks |= set(skipped.cpu().tolist()[:3])
        sample = torch.tensor(sorted(picks), dtype=torch.int64, device=DEV)
        q_before = W.as_u16(inp["q"].index_select(0, sample))
        op(inp["q"], inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"], slots_all,
           inp["cache"])
        torch.cuda.synchronize()
        note("  launched; checking %d sampled tokens" % sample.numel())
        q_after = W.as_u16(inp["q"].index_select(0, sample))
        kv = W.as_u16(inp["kv"].index_select(0, sample))
        pos = inp["positions"].index_select(0, sample).cpu().numpy()
        slots = slots_all.index_select(0, sample).cpu().numpy()
        cs = inp["cos_sin"].cpu().numpy()
        qw, kvw = W.as_u16(inp["q_w"]), W.as_u16(inp["kv_w"])
        B = w.block_size
        cap = w.num_blocks * B
        for i in range(sample.numel()):
            s = int(slots[i])
            valid = 0 <= s < cap
            one = np.zeros((1, B * qp.SLOT_BYTES), dtype=np.uint8)
            want_q = oracle.qkv_prep(q_before[i:i + 1], kv[i:i + 1], qw, kvw, pos[i:i + 1], cs,
                                     np.array([s % B if valid else -1], dtype=np.int64), one, 1, B, w.eps)
            assert np.array_equal(q_after[i], want_q[0]), "token %d: q differs" % int(sample[i])
            if valid:
                blk, sib = divmod(s, B)
                got = inp["cache"][blk].cpu().numpy()
                data = slice(sib * 576, sib * 576 + 576)
                rec = slice(B * 576 + sib * 8, B * 576 + sib * 8 + 8)
                assert np.array_equal(got[data], one[0, data]), "token %d: slot data differs" % int(sample[i])
                assert np.array_equal(got[rec], one[0, rec]), "token %d: scale record differs" % int(sample[i])
        note("  -> %d tokens bit-exact (%d skipped among them)" % (
            sample.numel(), int((slots < 0).sum())))
    finally:
        del inp
        torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reader_at_its_row_limit_on_sampled_rows(dtype):
    """2^26 - 1 rows, the most the reader takes.  For fp32 rows the grid's
    XCD padding would reach 2^32 work-items there, so the plain order runs;
    bf16 rows (two per wavefront) keep the padding.  Slots are drawn at random
    over a 262144-slot cache, some out of range; sampled rows are compared with
    the oracle's dequantization, bit for bit."""
    n = (1 << 26) - 1
    nb, bs = 4096, 64
    per = 4 if dtype == "f32" else 2
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    need = n * 512 * per + n * 8 + nb * bs * qp.SLOT_BYTES + (2 << 30)
    if need > free:
        pytest.skip("needs %.0f GB of free device memory, %.0f GB free" % (need / 1e9, free / 1e9))
    rng = np.random.default_rng(1200 + per)
    host = rng.integers(0, 256, (nb, bs * qp.SLOT_BYTES), dtype=np.uint8)
    data = host[:, :bs * 576]
    data[(data & 0x7F) == 0x7F] -= 1                     # no NaN codes: 0x7F -> 0x7E, 0xFF -> 0xFE
    host[:, bs * 576:] = rng.integers(100, 140, (nb, bs * 8), dtype=np.uint8)
    cache = torch.from_numpy(host).to(DEV)
    gen = torch.Generator(device=DEV).manual_seed(1201)
    slots = torch.randint(-3, nb * bs + 3, (n,), dtype=torch.int64, device=DEV, generator=gen)
    out = torch.empty((n, 512), dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device=DEV)
    try:
        note("reader %s: %d rows (%.0f GB out)" % (dtype, n, out.numel() * out.element_size() / 1e9))
        qp.QkvPrep(64, block_size=bs).gather(cache, slots, out)
        torch.cuda.synchronize()
        bad = torch.nonzero((slots < 0) | (slots >= nb * bs)).flatten()[:4].cpu().tolist()
        picks = sorted(set(rng.choice(n, 200, replace=False).tolist()) | {0, 1, n - 2, n - 1} | set(bad))
        idx = torch.tensor(picks, dtype=torch.int64, device=DEV)
        s = slots.index_select(0, idx).cpu().numpy()
        want = oracle.gather_dequant(host, nb, bs, s)
        got = out.index_select(0, idx)
        if dtype == "f32":
            assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))
        else:
            assert np.array_equal(W.as_u16(got), oracle.f32_to_bf16(want))
        note("  -> %d sampled rows bit-exact (%d out of range)" % (len(picks), int(((s < 0) | (s >= nb * bs)).sum())))
    finally:
        del out, slots, cache
        torch.cuda.empty_cache()


def _tile_check(x, r, gamma, eps, codes, scales, res_out, m, hidden, tile):
    """Rows of one 128-row tile against the oracle: codes, the tile's block
    of swizzled scales (laid out as for a batch of one tile), residual out."""
    r0, r1 = tile * 128, min(m, tile * 128 + 128)
    cols = hidden // 32
    xh = W.as_u16(x[r0:r1])
    rh = None if r is None else W.as_u16(r[r0:r1])
    want_codes, want_scales, want_res = oracle.mxfp8_norm_quant(xh, W.as_u16(gamma), eps, residual=rh)
    assert np.array_equal(codes[r0:r1].cpu().numpy(), want_codes), "tile %d: codes" % tile
    got_scales = scales[tile * 128 * cols:(tile + 1) * 128 * cols].cpu().numpy()
    assert np.array_equal(got_scales, want_scales), "tile %d: scales" % tile
    if res_out is not None:
        assert np.array_equal(W.as_u16(res_out[r0:r1]), want_res), "tile %d: residual out" % tile


@pytest.mark.timeout(900)
@pytest.mark.parametrize("hidden,lanes,res_out", [(128, 64, True), (1152, 192, False)])
def test_mxfp8_at_its_grid_limit_on_sampled_tiles(hidden, lanes, res_out):
    """The most rows the MXFP8 operator takes at two row widths whose
    workgroup has more lanes than the row has 16-byte chunks (64 for 16 at
    hidden 128, 192 for 144 at hidden 1152): round_up(m, 128) workgroups just
    below 2^32 work-items, with a ragged last tile.  Sampled 128-row tiles
    (the first, the last, random ones) are compared with the oracle."""
    top = (2 ** 32 - 1) // lanes // 128 * 128
    m = top - 37
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    need = m * hidden * (2 + 2 + (2 if res_out else 0) + 1) + top * hidden // 32 + (2 << 30)
    if need > free:
        pytest.skip("needs %.0f GB of free device memory, %.0f GB free" % (need / 1e9, free / 1e9))
    gen = torch.Generator(device=DEV).manual_seed(1300 + hidden)
    x = torch.empty((m, hidden), dtype=torch.bfloat16, device=DEV)
    r = torch.empty_like(x)
    step = 1 << 20
    for i in range(0, m, step):
        x[i:i + step] = torch.randn((min(step, m - i), hidden), generator=gen, device=DEV).to(torch.bfloat16)
        r[i:i + step] = torch.randn((min(step, m - i), hidden), generator=gen, device=DEV).to(torch.bfloat16)
    gamma = (0.1 * torch.randn(hidden, generator=gen, device=DEV)).to(torch.bfloat16)
    ro = torch.empty_like(x) if res_out else None
    try:
        note("mxfp8 %d x %d (x %.0f GB), residual out %s" % (m, hidden, x.numel() * 2 / 1e9, res_out))
        codes, scales = qp.mxfp8_norm_quant(x, gamma, 1e-6, residual=r, residual_out=ro)
        torch.cuda.synchronize()
        assert scales.numel() == top * hidden // 32
        last = (m - 1) // 128
        rng = np.random.default_rng(hidden)
        tiles = sorted(set(rng.choice(last, 6, replace=False).tolist()) | {0, last})
        for t in tiles:
            _tile_check(x, r, gamma, 1e-6, codes, scales, ro, m, hidden, t)
        note("  -> %d sampled tiles bit-exact" % len(tiles))
    finally:
        del x, r, ro
        torch.cuda.empty_cache()
