"""Pins of the oracle's number formats (bf16, E4M3, UE8M0) against things other
than the oracle itself: hand-derived values (tests/golden), torch's own casts
(a library routine), a nearest-value search written from the format
definitions, and exact comparisons in float64."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_known_values.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _f32(s):
    return np.float32(float(s))


# ------------------------------------------------------------------- bf16

def test_bf16_known_values():
    for case in _golden()["bf16"]["cases"]:
        got = int(oracle.f32_to_bf16(np.array([_f32(case["value"])]))[0])
        assert got == int(case["bits"], 16), case


def test_bf16_matches_torch_cast_on_strided_patterns():
    # Every 97th fp32 bit pattern (97 is odd, so every residue class of the
    # dropped 16 bits is visited), NaNs aside.
    bits = np.arange(0, 2 ** 32, 97, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    ours = oracle.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_ties_and_neighbours_exhaustive():
    # For every finite bf16 magnitude b: the exact midpoint to the next bf16 and
    # the fp32 values one ulp either side of it.
    hi = np.arange(0, 0x7f80, dtype=np.uint32)
    mid = (hi << 16) | 0x8000
    x = np.concatenate([mid, mid - 1, mid + 1]).view(np.float32)
    x = np.concatenate([x, -x])
    ours = oracle.f32_to_bf16(x)
    # Nearest-value search from the definition, in float64: candidates are the
    # truncation and the next bf16 up; ties pick the even pattern.
    u = x.view(np.uint32)
    mag = u & 0x7FFFFFFF
    lo = mag & 0xFFFF0000
    up = lo + 0x10000
    v = np.abs(x.astype(np.float64))
    dlo = v - lo.view(np.float32).astype(np.float64)
    upv = np.where(up == 0x7F800000, 2.0 ** 128, up.view(np.float32).astype(np.float64))
    dup = upv - v
    pick_up = (dup < dlo) | ((dup == dlo) & (((lo >> 16) & 1) == 1))
    want = (np.where(pick_up, up, lo) | (u & 0x80000000)) >> 16
    assert np.array_equal(ours, want.astype(np.uint16))


# ------------------------------------------------------------------- E4M3

def test_e4m3_known_values():
    for case in _golden()["e4m3"]["cases"]:
        got = int(oracle.f32_to_e4m3(np.array([_f32(case["value"])]))[0])
        assert got == int(case["code"], 16), case


def test_e4m3_decode_table():
    # Every code decodes to the e4m3fn value; 0x7f/0xff are NaN; the positive
    # codes are strictly increasing.
    vals = oracle.e4m3_to_f64(np.arange(256))
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert pos[0] == 0.0 and pos[1] == 2.0 ** -9 and pos[8] == 2.0 ** -6 and pos[0x7E] == 448.0
    assert np.array_equal(vals[0x80:0xFF], -pos)


def test_e4m3_round_trip_every_code():
    vals = oracle.e4m3_to_f64(np.arange(256))
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    again = oracle.f32_to_e4m3(vals[codes].astype(np.float32))
    assert np.array_equal(again, codes.astype(np.uint8))


def _over_chunks(fn, lo, hi, chunk=1 << 24):
    """fn(start, stop) over [lo, hi) in chunks, on a thread pool (the oracle's
    C loops and torch's casts release the GIL).  Returns the failing starts."""
    from concurrent.futures import ThreadPoolExecutor
    starts = range(lo, hi, chunk)
    with ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
        ok = list(ex.map(lambda s: fn(s, min(s + chunk, hi)), starts))
    return [hex(s) for s, good in zip(starts, ok) if not good]


def test_e4m3_matches_torch_cast_on_every_in_range_pattern():
    # Every fp32 bit pattern of magnitude up to 448 (0 .. 0x43E00000), both
    # signs: about 2.3e9 values.  Inside this range torch's float8_e4m3fn cast
    # is plain round-to-nearest-even.
    def check(start, stop):
        x = np.arange(start, stop, dtype=np.uint32).view(np.float32)
        x = np.concatenate([x, -x])
        ours = oracle.f32_to_e4m3(x)
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        return np.array_equal(ours, ref)
    assert _over_chunks(check, 0, 0x43E00001) == []


def test_e4m3_nearest_search_on_random_values():
    # Nearest code by brute force over the 127 non-negative finite codes, ties
    # to the even mantissa (even code), values above 448 saturated.
    rng = np.random.default_rng(5)
    mags = np.concatenate([
        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), 20000)),
        rng.uniform(0, 2.0 ** -6, 5000),
    ]).astype(np.float32)
    x = np.concatenate([mags, -mags])
    ours = oracle.f32_to_e4m3(x)
    table = oracle.e4m3_to_f64(np.arange(0x7F))
    a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    d = np.abs(a[:, None] - table[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    idx = np.where(cand.sum(axis=1) > 1, np.argmax(cand & (np.arange(0x7F) % 2 == 0), axis=1),
                   np.argmax(cand, axis=1))
    want = idx.astype(np.uint8) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    assert np.array_equal(ours, want)


# ------------------------------------------------------------------- UE8M0

def test_ue8m0_known_values():
    cases = _golden()["ue8m0"]["cases"]
    a = np.array([_f32(c["amax"]) for c in cases], np.float32)
    got = oracle.ue8m0_exponent(a) + 127
    assert [int(v) for v in got] == [c["byte"] for c in cases]


def test_ue8m0_definition_on_random_patterns():
    rng = np.random.default_rng(11)
    bits = rng.integers(1, 0x7F800000, 200000, dtype=np.uint32)   # positive finite
    a = bits.view(np.float32)
    e = oracle.ue8m0_exponent(a).astype(np.int64)
    av = a.astype(np.float64)
    assert np.all((e >= -127) & (e <= 127))
    fits = av <= 448.0 * np.ldexp(1.0, e)
    assert np.all(fits)
    # minimal, except where the clamp at -127 is active
    prev_fits = av <= 448.0 * np.ldexp(1.0, e - 1)
    assert not np.any(prev_fits & (e > -127))
    # the scale is an exact power of two and every scaled value fits 448
    assert np.all(np.abs(av * np.ldexp(1.0, -e)) <= 448.0)


def test_ue8m0_definition_on_every_positive_pattern():
    # Every positive finite fp32 amax (about 2.1e9 patterns): the exponent is
    # in [-127, 127], amax fits 448 * 2^e, and e - 1 would not fit unless the
    # clamp at -127 is active.  Comparisons are exact in float64.
    def check(start, stop):
        a = np.arange(start, stop, dtype=np.uint32).view(np.float32)
        e = oracle.ue8m0_exponent(a).astype(np.int64)
        av = a.astype(np.float64)
        return bool(np.all((e >= -127) & (e <= 127)) and np.all(av <= np.ldexp(448.0, e)) and
                    not np.any((av <= np.ldexp(448.0, e - 1)) & (e > -127)))
    assert _over_chunks(check, 1, 0x7F800000) == []


def test_ue8m0_power_of_two_boundaries():
    k = np.arange(-100, 100)
    at = (448.0 * np.ldexp(1.0, k)).astype(np.float32)
    above = np.nextafter(at, np.float32(np.inf))
    below = np.nextafter(at, np.float32(0))
    assert np.array_equal(oracle.ue8m0_exponent(at), k)
    assert np.array_equal(oracle.ue8m0_exponent(above), k + 1)
    assert np.array_equal(oracle.ue8m0_exponent(below), k)
