"""GPU checks that every entry point writes only its outputs.  Each output
tensor is a view into a larger device buffer whose bytes before and after it
hold a seeded pattern; after the call those guard bytes must be unchanged, and
the output itself must equal the same call's output on ordinary tensors (which
the parity tests check against the oracle).  The stores go through buffer
descriptors built from per-row or per-slot base addresses, so a wrong base or
range would show here as a changed guard byte."""
import pytest
import torch

from fp8_kv_cache_amd import probe
from fp8_kv_cache_amd import qkv_prep as qp
from fp8_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GUARD = 4096


class Guarded:
    """`nbytes` of output space between two GUARD-byte bands of a seeded
    pattern (the band edges stay 16-byte aligned)."""

    def __init__(self, nbytes, seed):
        g = torch.Generator(device=DEV).manual_seed(seed)
        self.nbytes = nbytes
        self.buf = torch.randint(0, 256, (GUARD + nbytes + GUARD,), dtype=torch.uint8, device=DEV,
                                 generator=g)
        self.before = None

    def view(self, dtype, shape):
        return self.buf[GUARD:GUARD + self.nbytes].view(dtype).view(shape)

    def arm(self):
        """Snapshot the guard bands once the output region holds its start values."""
        torch.cuda.synchronize()
        self.before = self.buf.clone()

    def assert_intact(self, what):
        torch.cuda.synchronize()
        end = GUARD + self.nbytes
        assert torch.equal(self.buf[:GUARD], self.before[:GUARD]), "%s: bytes before the output changed" % what
        assert torch.equal(self.buf[end:], self.before[end:]), "%s: bytes after the output changed" % what


def same_bytes(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("T,H,rpw,kv_store", [
    (1, 1, 0, qp.KV_FP8), (777, 5, 1, qp.KV_FP8), (777, 5, 2, qp.KV_FP8), (300, 64, 0, qp.KV_FP8),
    (4096, 64, 1, qp.KV_FP8), (300, 8, 1, qp.KV_BF16), (300, 8, 2, qp.KV_BF16),
    (2051, 64, 0, qp.KV_FP8), (2051, 64, 0, qp.KV_BF16),    # four tokens per kv wavefront, ragged
    (29131, 9, 0, qp.KV_FP8)])                              # kv workgroups spread through the grid
def test_operator_writes_only_q_and_the_cache(T, H, rpw, kv_store):
    w = W.custom(T, H, seed=1300 + T + H, num_skip=min(T // 4, 5))
    inp = W.make_inputs(w, device=DEV)
    slot_bytes = qp.SLOT_BYTES if kv_store == qp.KV_FP8 else qp.BF16_SLOT_BYTES
    g = torch.Generator(device=DEV).manual_seed(w.seed + 5)
    cache0 = torch.randint(0, 256, (w.num_blocks, w.block_size * slot_bytes), dtype=torch.uint8,
                           device=DEV, generator=g)
    op = qp.QkvPrep(H, block_size=w.block_size, eps=w.eps, rows_per_wave=rpw, kv_store=kv_store)
    if T * H >= 1 << 16:
        assert op.launch_shape(T).kv_per_wave == 4
    rest = (inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"], inp["slot_mapping"])

    q_ref, cache_ref = inp["q"].clone(), cache0.clone()
    op(q_ref, *rest, cache_ref)

    gq = Guarded(T * H * 1024, seed=w.seed + 1)
    q = gq.view(torch.bfloat16, (T, H, 512))
    q.copy_(inp["q"])
    gq.arm()
    gc = Guarded(cache0.numel(), seed=w.seed + 2)
    cache = gc.view(torch.uint8, tuple(cache0.shape))
    cache.copy_(cache0)
    gc.arm()
    op(q, *rest, cache)
    gq.assert_intact("q")
    gc.assert_intact("cache")
    assert same_bytes(q, q_ref)
    assert same_bytes(cache, cache_ref)


@pytest.mark.parametrize("dtype,drop", [(torch.float32, 0), (torch.bfloat16, 0), (torch.float32, 1),
                                        (torch.bfloat16, 1), (torch.bfloat16, 999)])
def test_gather_writes_only_its_rows(dtype, drop):
    # drop = 1 leaves an odd row count, so the last two-row bf16 wavefront has
    # one row to write; drop = 999 leaves a single row.
    w = W.custom(1000, 4, seed=1400, num_skip=7)
    inp = W.make_inputs(w, device=DEV)
    op = qp.QkvPrep(4, block_size=w.block_size, eps=w.eps)
    op(inp["q"], inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"], inp["slot_mapping"],
       inp["cache"])
    slots = inp["slot_mapping"].flip(0)[drop:].contiguous()   # includes the skipped (negative) slots
    n = slots.numel()
    ref = torch.empty((n, 512), dtype=dtype, device=DEV)
    op.gather(inp["cache"], slots, ref)
    gout = Guarded(n * 512 * ref.element_size(), seed=1401)
    out = gout.view(dtype, (n, 512))
    gout.arm()
    op.gather(inp["cache"], slots, out)
    gout.assert_intact("gather out")
    assert same_bytes(out, ref)


@pytest.mark.parametrize("m,hidden", [(130, 1024), (3, 7168), (1, 512)])
def test_mxfp8_writes_only_its_outputs(m, hidden):
    g = torch.Generator(device=DEV).manual_seed(1500 + m)
    x = torch.randn((m, hidden), generator=g, device=DEV).to(torch.bfloat16)
    r = torch.randn((m, hidden), generator=g, device=DEV).to(torch.bfloat16)
    gamma = (0.1 * torch.randn(hidden, generator=g, device=DEV)).to(torch.bfloat16)
    nsc = qp.qkv_prep_mxfp8_scale_bytes(m, hidden)
    ref_res = torch.empty_like(x)
    ref_codes, ref_scales = qp.mxfp8_norm_quant(x, gamma, 1e-6, residual=r, residual_out=ref_res)

    gcodes, gscales, gres = Guarded(m * hidden, 1501), Guarded(nsc, 1502), Guarded(m * hidden * 2, 1503)
    codes = gcodes.view(torch.uint8, (m, hidden))
    scales = gscales.view(torch.uint8, (nsc,))
    res = gres.view(torch.bfloat16, (m, hidden))
    for gz in (gcodes, gscales, gres):
        gz.arm()
    qp.mxfp8_norm_quant(x, gamma, 1e-6, residual=r, residual_out=res, quant_out=codes, scale_out=scales)
    gcodes.assert_intact("codes")
    gscales.assert_intact("scales")
    gres.assert_intact("residual_out")
    torch.cuda.synchronize()
    assert same_bytes(codes, ref_codes) and same_bytes(scales, ref_scales) and same_bytes(res, ref_res)


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16 * 37])
def test_probes_write_only_their_buffers(nbytes):
    st = torch.cuda.current_stream().cuda_stream
    g = torch.Generator(device=DEV).manual_seed(1600 + nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    gd = Guarded(nbytes, 1601)
    dst = gd.view(torch.uint8, (nbytes,))
    gd.arm()
    probe.qkv_prep_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, st)
    gd.assert_intact("probe copy")
    assert torch.equal(dst, src)
    gu = Guarded(nbytes, 1602)
    buf = gu.view(torch.uint8, (nbytes,))
    gu.arm()
    start = buf.clone()
    probe.qkv_prep_probe_update(buf.data_ptr(), nbytes, st)
    gu.assert_intact("probe update")
    want = start.view(torch.int32).clone()
    want[0::4] += 1                                  # word 0 of every 16-byte chunk, wrapping
    assert torch.equal(buf.view(torch.int32), want)


def _slot_byte_mask(slots, num_blocks, block_size, kv_store):
    """Host mask of the cache bytes the operator may write for these slots:
    the data and scale records of every valid slot (FP8 layout), or the
    1024-byte slot (bf16 layout)."""
    import numpy as np
    slot_bytes = qp.SLOT_BYTES if kv_store == qp.KV_FP8 else qp.BF16_SLOT_BYTES
    mask = np.zeros(num_blocks * block_size * slot_bytes, bool)
    for s in slots:
        if not 0 <= s < num_blocks * block_size:
            continue
        if kv_store == qp.KV_BF16:
            mask[s * 1024:(s + 1) * 1024] = True
            continue
        b, i = divmod(int(s), block_size)
        base = b * block_size * qp.SLOT_BYTES
        mask[base + i * 576: base + (i + 1) * 576] = True
        mask[base + block_size * 576 + i * 8: base + block_size * 576 + (i + 1) * 8] = True
    return mask


@pytest.mark.parametrize("T,H,kv_store", [(300, 8, qp.KV_FP8), (300, 8, qp.KV_BF16),
                                          (2051, 64, qp.KV_FP8), (2051, 64, qp.KV_BF16)])
def test_non_finite_rows_write_only_their_own_spans(T, H, kv_store):
    # Non-finite inputs are outside the numerics contract, so their values are
    # not checked; what must still hold is that such rows (whole rows of NaN,
    # of +-inf, single NaN or inf elements, rows whose sum of squares
    # overflows) write only their own q row and their own cache slot.  Guard
    # bands surround q and the cache, and every cache byte outside the valid
    # slots' records must keep its value.
    import numpy as np
    note = "non-finite rows: T=%d H=%d kv_store=%d" % (T, H, kv_store)
    print(note, flush=True)
    w = W.custom(T, H, seed=1600 + T + kv_store, num_skip=7)
    inp = W.make_inputs(w, device=DEV)
    q_src, kv_src = inp["q"].clone(), inp["kv"].clone()
    nan, inf = float("nan"), float("inf")
    q_src[::7, 0, :] = nan
    q_src[1::7, H - 1, :] = inf
    q_src[2::7, H // 2, 5] = nan
    q_src[3::7, 0, 450] = -inf
    q_src[4::11, :, :] = 3.0e38                      # finite, but the squares overflow
    kv_src[::5, :] = nan
    kv_src[1::5, 100] = inf
    kv_src[2::5, 460] = nan
    kv_src[3::5, :] = -inf
    rest = (kv_src, inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"], inp["slot_mapping"])
    slot_bytes = qp.SLOT_BYTES if kv_store == qp.KV_FP8 else qp.BF16_SLOT_BYTES
    g = torch.Generator(device=DEV).manual_seed(w.seed + 5)
    cache0 = torch.randint(0, 256, (w.num_blocks, w.block_size * slot_bytes), dtype=torch.uint8,
                           device=DEV, generator=g)
    op = qp.QkvPrep(H, block_size=w.block_size, eps=w.eps, kv_store=kv_store)
    gq = Guarded(T * H * 1024, seed=w.seed + 1)
    q = gq.view(torch.bfloat16, (T, H, 512))
    q.copy_(q_src)
    gq.arm()
    gc = Guarded(cache0.numel(), seed=w.seed + 2)
    cache = gc.view(torch.uint8, tuple(cache0.shape))
    cache.copy_(cache0)
    gc.arm()
    op(q, *rest, cache)
    gq.assert_intact("q")
    gc.assert_intact("cache")
    mask = _slot_byte_mask(inp["slot_mapping"].cpu().numpy(), w.num_blocks, w.block_size, kv_store)
    after = cache.cpu().numpy().reshape(-1)
    before = cache0.cpu().numpy().reshape(-1)
    assert np.array_equal(after[~mask], before[~mask]), "bytes outside the valid slots changed"
