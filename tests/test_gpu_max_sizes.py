"""The largest batches one MI355X holds, at the sizes where the launch
heuristic's grid-size fallbacks take over: from 2^26 q rows a wavefront per
row would pass 2^32 work-items, so two heads share a wavefront, and from about
1.3e8 rows four do.  q alone is 78 GB and 144 GB here.  Every token cannot be
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
@pytest.mark.parametrize("T,H,rows_per_wave", [(600000, 128, 2), (1100000, 128, 4)])
def test_largest_batches_on_sampled_tokens(T, H, rows_per_wave):
    w = W.custom(T, H, seed=T // 1000 + H, num_skip=7)
    need = T * H * 1024 + T * 1024 + w.num_blocks * w.block_size * qp.SLOT_BYTES + (2 << 30)
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if need > free:
        pytest.skip("needs %.0f GB of free device memory, %.0f GB free" % (need / 1e9, free / 1e9))
    op = qp.QkvPrep(H, block_size=w.block_size, eps=w.eps)
    shape = op.launch_shape(T)
    assert shape.rows_per_wave == rows_per_wave
    assert (shape.kv_blocks + shape.q_blocks) * 64 < 2 ** 32
    note("case %s: drawing inputs (q %.0f GB), launch %s" % (
        w.label, T * H * 1024 / 1e9, (shape.rows_per_wave, shape.kv_per_wave, shape.grid)))
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
