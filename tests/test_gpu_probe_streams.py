"""GPU checks of the policy-selectable stream probe (qkv_prep_probe_stream):
for every stream kind, accepted cache policy, pause, workgroup size and
number of chunks per lane, on ragged sizes, the probe computes what its header
states and writes nothing outside its range (seeded guard bands around every
written buffer).  The cache-policy bits change where lines are kept, never the
bytes written, so every policy must give the same result."""
import itertools

import numpy as np
import pytest
import torch

from fp8_kv_cache_amd import probe

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GUARD = 4096
LANES = (64, 128, 256, 512, 1024)
LOADS = (0, probe.NT, probe.NT | probe.SC1)
STORES = (0, probe.NT, probe.SC1, probe.NT | probe.SC1, probe.SC0 | probe.NT | probe.SC1)
# Chunk counts: below one workgroup, ragged over several, and exact multiples.
CHUNKS = (1, 63, 1000, 4096, 70001)


def guarded(nbytes, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randint(0, 256, (GUARD + nbytes + GUARD,), dtype=torch.uint8, device=DEV, generator=g)


def check_guards(buf, before, nbytes, what):
    torch.cuda.synchronize()
    assert torch.equal(buf[:GUARD], before[:GUARD]), "%s: bytes before the range changed" % what
    assert torch.equal(buf[GUARD + nbytes:], before[GUARD + nbytes:]), "%s: bytes after the range changed" % what


def stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("chunks", CHUNKS)
def test_write_stream_pattern_every_policy(chunks):
    nbytes = chunks * 16
    key = 0x1234ABCD
    i = np.arange(chunks, dtype=np.uint64)
    want = np.stack([(i & 0xFFFFFFFF).astype(np.uint32), (i >> np.uint64(32)).astype(np.uint32),
                     np.full(chunks, key, np.uint32), np.full(chunks, ~np.uint32(key), np.uint32)], axis=1)
    for n, (sp, lanes) in enumerate(itertools.product(STORES, LANES)):
        buf = guarded(nbytes, 100 + n)
        before = buf.clone()
        probe.qkv_prep_probe_stream(probe.WRITE, 0, sp, 0, lanes, 1, 0, buf[GUARD:].data_ptr(), None, nbytes, key,
                                    stream())
        what = "write chunks=%d store=%d lanes=%d" % (chunks, sp, lanes)
        check_guards(buf, before, nbytes, what)
        got = buf[GUARD:GUARD + nbytes].cpu().numpy().view(np.uint32).reshape(chunks, 4)
        assert np.array_equal(got, want), what


@pytest.mark.parametrize("chunks", CHUNKS)
def test_copy_stream_every_policy(chunks):
    nbytes = chunks * 16
    g = torch.Generator(device=DEV).manual_seed(chunks)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    for n, (lp, sp, sleep, lanes) in enumerate(itertools.product(LOADS, STORES, (0, 1), LANES)):
        if lanes not in (64, 256, 1024) and (lp, sp) != (probe.NT, probe.NT | probe.SC1):
            continue
        buf = guarded(nbytes, 200 + n)
        before = buf.clone()
        probe.qkv_prep_probe_stream(probe.COPY, lp, sp, sleep, lanes, 1, 0, buf[GUARD:].data_ptr(), src.data_ptr(),
                                    nbytes, 0, stream())
        what = "copy chunks=%d load=%d store=%d sleep=%d lanes=%d" % (chunks, lp, sp, sleep, lanes)
        check_guards(buf, before, nbytes, what)
        assert torch.equal(buf[GUARD:GUARD + nbytes], src), what


@pytest.mark.parametrize("chunks", CHUNKS)
def test_update_stream_every_policy(chunks):
    nbytes = chunks * 16
    for n, (lp, sp, sleep, lanes) in enumerate(itertools.product(LOADS, STORES, (0, 1), LANES)):
        if lanes not in (64, 256, 1024) and (lp, sp) != (probe.NT, probe.NT | probe.SC1):
            continue
        buf = guarded(nbytes, 300 + n)
        words = buf[GUARD:GUARD + nbytes].view(torch.int32).view(chunks, 4)
        words[::5, 0] = -1                         # 0xFFFFFFFF wraps to 0
        before = buf.clone()
        probe.qkv_prep_probe_stream(probe.UPDATE, lp, sp, sleep, lanes, 1, 0, buf[GUARD:].data_ptr(), None, nbytes, 0,
                                    stream())
        what = "update chunks=%d load=%d store=%d sleep=%d lanes=%d" % (chunks, lp, sp, sleep, lanes)
        check_guards(buf, before, nbytes, what)
        old = before[GUARD:GUARD + nbytes].cpu().numpy().view(np.uint32).reshape(chunks, 4)
        got = buf[GUARD:GUARD + nbytes].cpu().numpy().view(np.uint32).reshape(chunks, 4)
        assert np.array_equal(got[:, 0], old[:, 0] + np.uint32(1)), what
        assert np.array_equal(got[:, 1:], old[:, 1:]), what


@pytest.mark.parametrize("chunks", CHUNKS)
def test_read_stream_writes_the_key_only_on_a_match(chunks):
    nbytes = chunks * 16
    key = 0x0BADF00D
    g = torch.Generator(device=DEV).manual_seed(7 + chunks)
    src = torch.randint(0, 1 << 30, (chunks, 4), dtype=torch.int32, device=DEV, generator=g)
    # Make no chunk XOR to the key, then plant the key in one chunk (the last
    # one: the ragged tail of the last workgroup).
    x = src[:, 0] ^ src[:, 1] ^ src[:, 2] ^ src[:, 3]
    src[x == key, 0] ^= 1
    for lp, lanes in itertools.product(LOADS, LANES):
        sink = torch.full((4,), 77, dtype=torch.int32, device=DEV)
        probe.qkv_prep_probe_stream(probe.READ, lp, 0, 0, lanes, 1, 0, sink.data_ptr(), src.data_ptr(), nbytes, key,
                                    stream())
        assert sink.tolist() == [77] * 4, "read without a match wrote the sink (load=%d lanes=%d)" % (lp, lanes)
    planted = src.clone()
    planted[-1, 3] = planted[-1, 0] ^ planted[-1, 1] ^ planted[-1, 2] ^ key
    for lp, lanes in itertools.product(LOADS, LANES):
        sink = torch.full((4,), 77, dtype=torch.int32, device=DEV)
        probe.qkv_prep_probe_stream(probe.READ, lp, 0, 0, lanes, 1, 0, sink.data_ptr(), planted.data_ptr(), nbytes,
                                    key, stream())
        assert sink.tolist() == [key, 77, 77, 77], "read with a match (load=%d lanes=%d)" % (lp, lanes)


DEPTHS = (2, 4, 8, 16)


@pytest.mark.parametrize("chunks", CHUNKS)
def test_streams_by_chunks_per_lane_and_xcd_order(chunks):
    """Every lane takes `depth` chunks, the workgroup's range is lanes * depth
    chunks and the last workgroup is ragged; with the XCD-contiguous order the
    ranges are dealt to the workgroups in another order and the grid is padded
    to a multiple of 8 workgroups."""
    nbytes = chunks * 16
    key = 0x5EED5EED
    g = torch.Generator(device=DEV).manual_seed(1000 + chunks)
    src = torch.randint(0, 1 << 30, (chunks, 4), dtype=torch.int32, device=DEV, generator=g)
    x = src[:, 0] ^ src[:, 1] ^ src[:, 2] ^ src[:, 3]
    src[x == key, 0] ^= 1
    i = np.arange(chunks, dtype=np.uint64)
    want_write = np.stack([(i & 0xFFFFFFFF).astype(np.uint32), (i >> np.uint64(32)).astype(np.uint32),
                           np.full(chunks, key, np.uint32), np.full(chunks, ~np.uint32(key), np.uint32)], axis=1)
    NT, NTS = probe.NT, probe.NT | probe.SC1
    for n, (depth, lanes, XCD) in enumerate(itertools.product((1,) + DEPTHS, (64, 256, 1024), (0, 1))):
        what = "chunks=%d depth=%d lanes=%d xcd_order=%d" % (chunks, depth, lanes, XCD)
        buf = guarded(nbytes, 400 + n)
        before = buf.clone()
        probe.qkv_prep_probe_stream(probe.WRITE, 0, NTS, 0, lanes, depth, XCD, buf[GUARD:].data_ptr(), None, nbytes,
                                    key, stream())
        check_guards(buf, before, nbytes, "write " + what)
        got = buf[GUARD:GUARD + nbytes].cpu().numpy().view(np.uint32).reshape(chunks, 4)
        assert np.array_equal(got, want_write), "write " + what

        buf = guarded(nbytes, 500 + n)
        before = buf.clone()
        probe.qkv_prep_probe_stream(probe.COPY, NT, NTS, 0, lanes, depth, XCD, buf[GUARD:].data_ptr(), src.data_ptr(),
                                    nbytes, 0, stream())
        check_guards(buf, before, nbytes, "copy " + what)
        assert torch.equal(buf[GUARD:GUARD + nbytes].view(torch.int32).view(chunks, 4), src), "copy " + what

        buf = guarded(nbytes, 600 + n)
        before = buf.clone()
        probe.qkv_prep_probe_stream(probe.UPDATE, NT, NTS, 0, lanes, depth, XCD, buf[GUARD:].data_ptr(), None, nbytes,
                                    0, stream())
        check_guards(buf, before, nbytes, "update " + what)
        old = before[GUARD:GUARD + nbytes].cpu().numpy().view(np.uint32).reshape(chunks, 4)
        got = buf[GUARD:GUARD + nbytes].cpu().numpy().view(np.uint32).reshape(chunks, 4)
        assert np.array_equal(got[:, 0], old[:, 0] + np.uint32(1)), "update " + what
        assert np.array_equal(got[:, 1:], old[:, 1:]), "update " + what

        sink = torch.full((4,), 77, dtype=torch.int32, device=DEV)
        probe.qkv_prep_probe_stream(probe.READ, NT, 0, 0, lanes, depth, XCD, sink.data_ptr(), src.data_ptr(), nbytes,
                                    key, stream())
        assert sink.tolist() == [77] * 4, "read without a match " + what
        planted = src.clone()
        planted[-1, 3] = planted[-1, 0] ^ planted[-1, 1] ^ planted[-1, 2] ^ key
        probe.qkv_prep_probe_stream(probe.READ, NT, 0, 0, lanes, depth, XCD, sink.data_ptr(), planted.data_ptr(),
                                    nbytes, key, stream())
        assert sink.tolist() == [key, 77, 77, 77], "read with a match " + what


# ------------------------------------------------------------ MXFP8 pattern

MX_SHAPES = ((1, 512), (130, 1536), (200, 7168), (129, 16384))   # 1536: three groups, one per wavefront
MX_STREAMS = (15, 7, 1, 2, 4, 3, 6, 13, 10)


@pytest.mark.parametrize("m,hidden", MX_SHAPES)
def test_mxfp8_pattern_probe_writes_what_its_header_states(m, hidden):
    import oracle
    g = torch.Generator(device=DEV).manual_seed(m + hidden)
    x = torch.randint(-(1 << 31), 1 << 31, (m, hidden // 2), dtype=torch.int64, device=DEV, generator=g)
    x = x.to(torch.int32)
    r = torch.randint(-(1 << 31), 1 << 31, (m, hidden // 2), dtype=torch.int64, device=DEV,
                      generator=g).to(torch.int32)
    gamma = torch.randint(-(1 << 31), 1 << 31, (hidden // 2,), dtype=torch.int64, device=DEV,
                          generator=g).to(torch.int32)
    gw = gamma.cpu().numpy().view(np.uint32).reshape(hidden // 8, 4)
    nscale = probe_scale_bytes(m, hidden)
    pad_cols = hidden // 32
    # Scale positions: word j of row `row` covers columns 4j..4j+3; the oracle's
    # swizzle gives each column's byte.
    rows_padded = (m + 127) // 128 * 128
    where = np.array([[oracle.mxfp8_scale_offset(row, col, pad_cols) for col in range(pad_cols)]
                      for row in range(rows_padded)], dtype=np.int64)
    xw = x.cpu().numpy().view(np.uint32).reshape(m, hidden // 8, 4)
    rw = r.cpu().numpy().view(np.uint32).reshape(m, hidden // 8, 4)
    for streams in MX_STREAMS:
        what = "m=%d hidden=%d streams=%d" % (m, hidden, streams)
        res, cod, sca, bar = (streams & 1, streams & 2, streams & 4, streams & 8)
        ro = guarded(m * hidden * 2, 700 + streams)
        cd = guarded(m * hidden, 800 + streams)
        sc = guarded(nscale, 900 + streams)
        before = [t.clone() for t in (ro, cd, sc)]
        probe.qkv_prep_probe_mxfp8_pattern(x.data_ptr(), r.data_ptr(), gamma.data_ptr(), ro[GUARD:].data_ptr(),
                                           cd[GUARD:].data_ptr(), sc[GUARD:].data_ptr(), m, hidden, streams,
                                           stream())
        torch.cuda.synchronize()
        w = xw ^ rw if res else xw
        e = w[:, 0, 0][:, None] if bar else np.zeros((m, 1), np.uint32)
        for buf, old, n, on, name in ((ro, before[0], m * hidden * 2, res, "residual_out"),
                                      (cd, before[1], m * hidden, cod, "codes"),
                                      (sc, before[2], nscale, sca, "scales")):
            check_guards(buf, old, n, "%s %s" % (name, what))
            if not on:
                assert torch.equal(buf, old), "%s written without its stream (%s)" % (name, what)
        if res:
            got = ro[GUARD:GUARD + m * hidden * 2].cpu().numpy().view(np.uint32).reshape(m, hidden // 8, 4)
            assert np.array_equal(got, w), "residual_out " + what
        if cod:
            got = cd[GUARD:GUARD + m * hidden].cpu().numpy().view(np.uint32).reshape(m, hidden // 8, 2)
            assert np.array_equal(got[:, :, 0], w[:, :, 0] ^ w[:, :, 1] ^ gw[None, :, 0] ^ e), "codes word 0 " + what
            assert np.array_equal(got[:, :, 1], w[:, :, 2] ^ w[:, :, 3] ^ gw[None, :, 1]), "codes word 1 " + what
        if sca:
            got = sc[GUARD:GUARD + nscale].cpu().numpy()
            word = (w[:, 0::16, 0] ^ w[:, 0::16, 3] ^ gw[None, 0::16, 3] ^ e).astype(np.uint32)   # [m, cols / 4]
            want = np.zeros((rows_padded, pad_cols), np.uint8)
            want[:m] = word.view(np.uint8).reshape(m, pad_cols)                   # little-endian bytes
            assert np.array_equal(got[where], want), "scales " + what


def probe_scale_bytes(m, hidden):
    return (m + 127) // 128 * 128 * (hidden // 32)
