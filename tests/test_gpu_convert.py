"""Exhaustive checks of the device conversions against the oracle's encoders.
qkv_prep_probe_convert runs the operator's own conversion code
(qkvp::dev::pack_e4m3 / pack_bf16) on an array; both paths (integer rounding
and the gfx950 conversion instructions) are compared with oracle.f32_to_e4m3 /
oracle.f32_to_bf16:
  * E4M3: every fp32 bit pattern of magnitude <= 448 (the range the operator
    converts), both signs -- about 2.3e9 values;
  * bf16: every 97th fp32 bit pattern (NaNs aside) and every rounding tie with
    its two fp32 neighbours, both signs.
Inputs are made on each side independently from the bit patterns (arange), so
nothing the device computes feeds the oracle."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_amd import probe
from fp8_kv_cache_amd import qkv_prep as qp

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CHUNK = 1 << 25
SIGN = -(1 << 31)          # int32 with only the sign bit set


def note(msg):
    print(msg, flush=True)


def device_bits(start, stop, negative):
    x = torch.arange(start, stop, dtype=torch.int32, device=DEV)
    if negative:
        x = x | SIGN
    return x.view(torch.float32)


def host_bits(start, stop, negative):
    x = np.arange(start, stop, dtype=np.uint32)
    if negative:
        x = x | np.uint32(0x80000000)
    return x.view(np.float32)


def run_probe(x, convert, e4m3=True, bf16=True):
    n = x.numel()
    e = torch.empty(n, dtype=torch.uint8, device=DEV) if e4m3 else None
    b = torch.empty(n, dtype=torch.int16, device=DEV) if bf16 else None
    probe.qkv_prep_probe_convert(x.data_ptr(), n, None if e is None else e.data_ptr(),
                              None if b is None else b.data_ptr(), convert,
                              torch.cuda.current_stream().cuda_stream)
    return e, b


def test_e4m3_on_every_in_range_pattern():
    stop_all = 0x43E00001                       # 448.0 is 0x43E00000
    jobs = [(s, min(s + CHUNK, stop_all), neg) for s in range(0, stop_all, CHUNK) for neg in (False, True)]
    note("E4M3: %d chunks of up to %d patterns" % (len(jobs), CHUNK))
    with ThreadPoolExecutor(max_workers=8) as pool:
        for k in range(0, len(jobs), 8):
            batch = jobs[k:k + 8]
            want = [pool.submit(lambda j: oracle.f32_to_e4m3(host_bits(*j)), j) for j in batch]
            for (start, stop, neg), fut in zip(batch, want):
                n = stop - start
                pad = (-n) % 4
                x = device_bits(start, stop + pad, neg)     # padded to a multiple of 4
                ref = fut.result()
                for convert in (1, 2):
                    got, _ = run_probe(x, convert, bf16=False)
                    got = got[:n].cpu().numpy()
                    bad = np.nonzero(got != ref)[0]
                    assert bad.size == 0, "convert=%d start=%#x neg=%s first bad pattern %#x: got %#x want %#x" % (
                        convert, start, neg, start + int(bad[0]), got[bad[0]], ref[bad[0]])
            note("  chunks %d..%d bit-exact" % (k, k + len(batch) - 1))


def test_bf16_on_strided_patterns_and_every_tie():
    strided = np.arange(0, 2 ** 32, 97, dtype=np.uint64).astype(np.uint32)
    hi = np.arange(0, 0x7F80, dtype=np.uint32)
    mid = (hi << 16) | 0x8000
    ties = np.concatenate([mid, mid - 1, mid + 1])
    bits = np.concatenate([strided, ties, ties | np.uint32(0x80000000)])
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    x = np.concatenate([x, np.zeros((-x.size) % 4, np.float32)])
    note("bf16: %d values" % x.size)
    want = oracle.f32_to_bf16(x)
    xd = torch.from_numpy(x.copy()).to(DEV)                    # host bit patterns, not device results
    for convert in (1, 2):
        _, got = run_probe(xd, convert, e4m3=False)
        got = got.cpu().numpy().view(np.uint16)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, "convert=%d first bad input %#x: got %#x want %#x" % (
            convert, x[bad[0]].view(np.uint32), got[bad[0]], want[bad[0]])


def test_ue8m0_rules_on_every_non_negative_pattern():
    # Both UE8M0 rules as the operators' device code computes them
    # (qkv_prep_probe_ue8m0), against the oracle, on every finite
    # non-negative fp32 pattern (about 2.1e9 values): the main operator's
    # scale byte e + 127 of a block amax, and the MXFP8 operator's byte.  Then
    # the MXFP8 inverse scale of every byte.
    stop_all = 0x7F800000
    jobs = [(s, min(s + CHUNK, stop_all)) for s in range(0, stop_all, CHUNK)]
    note("UE8M0: %d chunks of up to %d patterns" % (len(jobs), CHUNK))

    def want(j):
        x = host_bits(j[0], j[1], False)
        return (oracle.ue8m0_exponent(x) + 127).astype(np.uint8), oracle.ue8m0_ceil_bytes(x)

    st = torch.cuda.current_stream().cuda_stream
    with ThreadPoolExecutor(max_workers=8) as pool:
        for k in range(0, len(jobs), 8):
            batch = jobs[k:k + 8]
            futs = [pool.submit(want, j) for j in batch]
            for (start, stop), fut in zip(batch, futs):
                n = stop - start
                x = device_bits(start, stop, False)
                op = torch.empty(n, dtype=torch.uint8, device=DEV)
                mx = torch.empty(n, dtype=torch.uint8, device=DEV)
                probe.qkv_prep_probe_ue8m0(x.data_ptr(), n, op.data_ptr(), mx.data_ptr(), None, st)
                want_op, want_mx = fut.result()
                for what, got, ref in (("operator byte", op, want_op), ("mxfp8 byte", mx, want_mx)):
                    got = got.cpu().numpy()
                    bad = np.nonzero(got != ref)[0]
                    assert bad.size == 0, "%s: first bad pattern %#x: got %d want %d" % (
                        what, start + int(bad[0]), got[bad[0]], ref[bad[0]])
            note("  chunks %d..%d bit-exact" % (k, k + len(batch) - 1))
    inv = torch.empty(256, dtype=torch.float32, device=DEV)
    probe.qkv_prep_probe_ue8m0(None, 0, None, None, inv.data_ptr(), st)
    got = inv.cpu().numpy()
    ref = np.array([oracle.ue8m0_inverse(b) for b in range(256)], np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
