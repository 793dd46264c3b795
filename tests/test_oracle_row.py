"""Pins of the oracle's per-row arithmetic: RMSNorm (sum-of-squares order,
inverse RMS, weight) and RoPE, against closed forms, invariants, hand-computed
cases and an independent float64 evaluation."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from fp8_kv_cache_amd.workloads import rope_table

F32_EPS = 2.0 ** -23


def bf16(x):
    return oracle.f32_to_bf16(np.asarray(x, np.float32))


def identity_cs(n=1):
    cs = np.zeros((n, 64), np.float32)
    cs[:, :32] = 1.0
    return cs


def rand_rows(n, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return bf16(rng.standard_normal((n, 512)) * scale)


# ------------------------------------------------------------- sum of squares

def _sumsq(x):
    buf = np.ascontiguousarray(x)             # keep the buffer alive across the call
    return float(oracle.lib().orc_sum_squares(buf.ctypes.data))


def test_sum_squares_hand_cases_pin_the_order():
    # The order: chunks of 8 summed left to right, then chunk sums added in
    # adjacent pairs over six levels.  4096^2 = 2^24, and 2^24 + 1 rounds to 2^24
    # (tie to even), so where the three extra ones meet 2^24 decides the sum.
    x = np.zeros(512, np.float32)
    x[0] = 4096.0
    x[8] = x[16] = x[24] = 1.0              # chunks 1, 2, 3
    # level 1: (2^24 + 1) -> 2^24 and (1 + 1) = 2; level 2: 2^24 + 2 (exact)
    assert _sumsq(bf16(x)) == 2.0 ** 24 + 2
    y = np.zeros(512, np.float32)
    y[0] = 4096.0
    y[2] = y[3] = 1.0                       # inside chunk 0, after 2^24
    # sequential inside the chunk: ((2^24 + 0) + 1) -> 2^24, (+ 1) -> 2^24
    assert _sumsq(bf16(y)) == 2.0 ** 24
    z = np.zeros(512, np.float32)
    z[0] = 4096.0
    z[256] = z[264] = 1.0                   # chunks 32 and 33
    # chunks 32 + 33 = 2 meet chunk 0's 2^24 only at the last level: 2^24 + 2
    assert _sumsq(bf16(z)) == 2.0 ** 24 + 2


def test_sum_squares_close_to_exact_sum():
    x = rand_rows(2000, 1)
    _, _, s, _ = oracle.rows(x, None, 1e-6, identity_cs(2000))
    exact = (oracle.bf16_to_f32(x).astype(np.float64) ** 2).sum(axis=1)
    # 7 sequential additions then 6 tree levels: relative error below 13 u.
    assert np.all(np.abs(s - exact) <= 13 * 2.0 ** -24 * exact)


# ------------------------------------------------------------- inverse RMS

def test_constant_power_of_two_row_closed_form():
    # A row of c = 2^k at eps = 0: S = 512 * 4^k exactly, mean 4^k, root 2^k,
    # so inv = 2^-k and every normalized value is exactly 1.
    for k in (-20, -3, 0, 5, 40):
        x = bf16(np.full((1, 512), 2.0 ** k))
        y, z, s, inv = oracle.rows(x, None, 0.0, identity_cs())
        assert s[0] == 512.0 * 4.0 ** k
        assert inv[0] == np.float32(2.0 ** -k)
        assert np.all(y == 1.0) and np.all(z == 1.0)


def test_power_of_two_scaling_leaves_outputs_unchanged():
    x = rand_rows(64, 2)
    w = bf16(1.0 + 0.1 * np.random.default_rng(3).standard_normal(512))
    cs = rope_table(4096)[np.random.default_rng(4).integers(0, 4096, 64)]
    y0, z0, _, _ = oracle.rows(x, w, 0.0, cs)
    for k in (-8, 3):
        xs = bf16(oracle.bf16_to_f32(x) * np.float32(2.0 ** k))
        y1, z1, _, _ = oracle.rows(xs, w, 0.0, cs)
        assert np.array_equal(y0, y1) and np.array_equal(z0, z1)


def test_zero_row_gives_zero():
    x = np.zeros((1, 512), np.uint16)
    y, z, s, inv = oracle.rows(x, bf16(np.ones(512)), 1e-6, identity_cs())
    assert s[0] == 0.0 and np.all(y == 0.0) and np.all(z == 0.0)
    assert inv[0] == np.float32(1.0) / np.sqrt(np.float32(1e-6))


def test_rms_of_unweighted_row_is_about_one():
    # RMS of x * inv is sqrt(ms / (ms + eps)), i.e. 1 up to eps and rounding.
    x = rand_rows(500, 5)
    eps = 1e-6
    y, _, s, _ = oracle.rows(x, None, eps, identity_cs(500))
    rms = np.sqrt((y.astype(np.float64) ** 2).mean(axis=1))
    ms = s.astype(np.float64) / 512
    assert np.all(np.abs(rms - np.sqrt(ms / (ms + eps))) < 1e-6)


def test_weighted_norm_against_float64():
    # y_j = x_j * inv * w_j evaluated in float64 from the same bf16 inputs:
    # the oracle's fp32 chain (sum, mean, add, sqrt, divide, two products)
    # stays within a few fp32 ulps of it.
    x = rand_rows(300, 6)
    w = bf16(1.0 + 0.1 * np.random.default_rng(7).standard_normal(512))
    eps = 1e-6
    y, _, _, _ = oracle.rows(x, w, eps, identity_cs(300))
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    wf = oracle.bf16_to_f32(w).astype(np.float64)
    ideal = xf / np.sqrt((xf ** 2).mean(axis=1, keepdims=True) + np.float64(np.float32(eps))) * wf
    assert np.all(np.abs(y - ideal) <= 12 * F32_EPS * np.abs(ideal) + 1e-30)


def test_constant_one_row_returns_the_weight():
    # x = 1 everywhere at eps = 0: inv = 1, so y = w bit for bit.
    w = bf16(1.0 + 0.1 * np.random.default_rng(8).standard_normal(512))
    y, z, _, inv = oracle.rows(bf16(np.ones((1, 512))), w, 0.0, identity_cs())
    assert inv[0] == 1.0
    assert np.array_equal(bf16(y[0]), w) and np.array_equal(bf16(z[0]), w)


# ------------------------------------------------------------- RoPE

def test_position_zero_is_identity():
    cs = rope_table(16)[:1]
    assert np.all(cs[0, :32] == 1.0) and np.all(cs[0, 32:] == 0.0)
    x = rand_rows(1, 9)
    y, z, _, _ = oracle.rows(x, None, 1e-6, cs)
    assert np.array_equal(y, z)


def test_rope_touches_only_its_pair_and_rotates_forward():
    # A one-hot at dim 448 must light dims 448 and 449 only (interleaved pairs,
    # not the first/second-half split), as (cos, sin) of the pair's angle.
    tab = rope_table(4096)
    p = 1234
    for i in (0, 5, 31):
        x = np.zeros((1, 512), np.float32)
        x[0, 448 + 2 * i] = 1.0
        y, z, _, _ = oracle.rows(bf16(x), None, 0.0, tab[p:p + 1])
        lit = np.nonzero(z[0])[0]
        assert set(lit.tolist()) <= {448 + 2 * i, 449 + 2 * i}
        # y[448+2i] = sqrt(512): scale out and compare with (cos, sin)
        a = y[0, 448 + 2 * i]
        c, s = tab[p, i], tab[p, 32 + i]
        assert z[0, 448 + 2 * i] == np.float32(a * c)
        assert z[0, 449 + 2 * i] == np.float32(a * s)
        x2 = np.zeros((1, 512), np.float32)
        x2[0, 449 + 2 * i] = 1.0
        y2, z2, _, _ = oracle.rows(bf16(x2), None, 0.0, tab[p:p + 1])
        b = y2[0, 449 + 2 * i]
        assert z2[0, 448 + 2 * i] == np.float32(-(b * s))
        assert z2[0, 449 + 2 * i] == np.float32(b * c)


def test_rope_preserves_pair_norm_and_matches_float64_rotation():
    rng = np.random.default_rng(12)
    tab = rope_table(131072)
    n = 400
    x = rand_rows(n, 13)
    cs = tab[rng.integers(0, 131072, n)]
    y, z, _, _ = oracle.rows(x, None, 1e-6, cs)
    a = y[:, 448::2].astype(np.float64)
    b = y[:, 449::2].astype(np.float64)
    c = cs[:, :32].astype(np.float64)
    s = cs[:, 32:].astype(np.float64)
    za, zb = z[:, 448::2].astype(np.float64), z[:, 449::2].astype(np.float64)
    n0 = a * a + b * b
    n1 = za * za + zb * zb
    table_err = np.abs(c * c + s * s - 1.0)
    assert np.all(np.abs(n1 - n0) <= (2.0 ** -21 + 2 * table_err) * n0 + 1e-30)
    ideal_a = a * c - b * s
    ideal_b = a * s + b * c
    mag = np.sqrt(n0)
    assert np.all(np.abs(za - ideal_a) <= 2 * F32_EPS * mag + 1e-30)
    assert np.all(np.abs(zb - ideal_b) <= 2 * F32_EPS * mag + 1e-30)
    # dims 0..447 are not rotated
    assert np.array_equal(y[:, :448], z[:, :448])


# ------------------------------------------------------------- rounding order
#
# The expected bits below are worked out in exact rational arithmetic
# (fractions.Fraction), with one explicit round-to-nearest-even to binary32
# per step of the stated formula, so they do not depend on how any float
# library orders or fuses its operations.  Each case is chosen so that the
# plausible alternative forms give different bits, which the test also checks:
# a case on which every form agrees pins nothing.

def rn32(x):
    """The binary32 value nearest to the rational x, ties to the even
    significand: 24 significant bits from 2^-126 up, a fixed quantum of 2^-149
    below it, and overflow to infinity once the rounded value reaches 2^128."""
    x = Fraction(x)
    if x == 0:
        return 0.0
    neg, m = x < 0, abs(x)
    e = m.numerator.bit_length() - m.denominator.bit_length()   # 2^e <= m < 2^(e+1), up to one step
    if Fraction(2) ** e > m:
        e -= 1
    elif Fraction(2) ** (e + 1) <= m:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    v = round(m / quantum) * quantum            # Fraction.__round__: ties to even
    if v >= Fraction(2) ** 128:
        return -math.inf if neg else math.inf
    return float(-v if neg else v)


def f32bits(v):
    return int(np.float32(v).view(np.uint32))


def test_rn32_helper_against_known_roundings():
    # The helper itself, on values whose binary32 rounding is known: ties to
    # even at 1 + 2^-24 and 1 + 3*2^-24, the smallest subnormal and the half of
    # it (a tie to zero), the overflow threshold, and one third.
    assert rn32(1 + Fraction(1, 2 ** 24)) == 1.0
    assert rn32(1 + Fraction(3, 2 ** 24)) == 1.0 + 2.0 ** -22
    assert rn32(Fraction(1, 2 ** 149)) == 2.0 ** -149
    assert rn32(Fraction(1, 2 ** 150)) == 0.0
    assert rn32(Fraction(3, 2 ** 150)) == 2.0 ** -148
    assert rn32(2 ** 128 - 2 ** 103) == math.inf
    assert rn32(2 ** 128 - 2 ** 103 - 1) == float(np.finfo(np.float32).max)
    assert f32bits(rn32(Fraction(1, 3))) == 0x3EAAAAAB
    assert f32bits(rn32(Fraction(-1, 7))) == 0xBE124925


def test_norm_product_order_row_of_sevens():
    # x = 7 in every dim, eps = 0: S = 512 * 49 = 25088 exactly, the mean is 49,
    # its root 7, so inv = RN(1/7) = 0x3E124925.  7 * RN(1/7) = 1 + 4.47e-8,
    # less than half an ulp (2^-24) above 1, so t = RN(x * inv) = 1 exactly and
    # the stated order y = RN(RN(x * inv) * w) returns the weight bit for bit.  The other
    # orders, RN(RN(x * w) * inv) and RN(x * RN(inv * w)), move about half of
    # these weights by an ulp.
    w = bf16(1.0 + 0.1 * np.random.default_rng(8).standard_normal(512))
    y, _, s, inv = oracle.rows(bf16(np.full((1, 512), 7.0)), w, 0.0, identity_cs())
    inv_exact = rn32(Fraction(1, 7))
    assert s[0] == 25088.0 and f32bits(inv[0]) == f32bits(inv_exact) == 0x3E124925
    assert rn32(7 * Fraction(inv_exact)) == 1.0
    wf = oracle.bf16_to_f32(w)
    assert np.array_equal(y[0].view(np.uint32), wf.view(np.uint32))
    inv_f = Fraction(inv_exact)
    weight_first = np.array([rn32(Fraction(rn32(7 * Fraction(float(v)))) * inv_f) for v in wf], np.float32)
    inv_w_first = np.array([rn32(7 * Fraction(rn32(inv_f * Fraction(float(v))))) for v in wf], np.float32)
    assert int((weight_first != wf).sum()) >= 100
    assert int((inv_w_first != wf).sum()) >= 100


def test_norm_product_order_exact_on_random_rows():
    # y_j = RN(RN(x_j * inv) * w_j) from the oracle's own inv (pinned by the
    # closed forms above) on random rows.  A product of two binary32 values has
    # at most 48 significant bits, so it is exact in binary64 and one
    # conversion to binary32 rounds it once: the expectation is exact.
    x = rand_rows(64, 21)
    w = bf16(1.0 + 0.1 * np.random.default_rng(22).standard_normal(512))
    y, _, _, inv = oracle.rows(x, w, 1e-6, identity_cs(64))
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    wf = oracle.bf16_to_f32(w).astype(np.float64)
    iv = inv.astype(np.float64)[:, None]
    t = (xf * iv).astype(np.float32).astype(np.float64)
    want = (t * wf).astype(np.float32)
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
    other = ((xf * wf).astype(np.float32).astype(np.float64) * iv).astype(np.float32)
    assert np.any(other != want)          # the case discriminates the orders


# Pair values found by search on the real table row of position 7 (angle 7 rad
# for pair 0): c = 0x3F40FFBD, s = 0x3F283046 (float32 cos 7, sin 7).
ROPE_C, ROPE_S = 0x3F40FFBD, 0x3F283046


def _f(bits):
    return float(np.uint32(bits).view(np.float32))


def test_rope_fma_form_hand_cases():
    # A row of ones at eps = 0 has inv = 1, so y = w exactly and the weight
    # sets the pair values.  Pair 0: (a, b) = (-0.875, -1.0625) checks the first
    # output a' = RN(a*c - RN(b*s)); pair 1: (a, b) = (1.25, -0.8125) checks the
    # second b' = RN(a*s + RN(b*c)).  Both pairs use c = cos 7, s = sin 7.
    c, s = _f(ROPE_C), _f(ROPE_S)
    w = np.ones(512, np.float32)
    w[448:452] = (-0.875, -1.0625, 1.25, -0.8125)
    cs = identity_cs()
    cs[0, 0] = cs[0, 1] = c
    cs[0, 32] = cs[0, 33] = s
    y, z, _, inv = oracle.rows(bf16(np.ones((1, 512))), bf16(w), 0.0, cs)
    assert inv[0] == 1.0 and np.array_equal(y[0], w)
    C, S = Fraction(c), Fraction(s)
    a, b = Fraction(-0.875), Fraction(-1.0625)
    first = {"pinned": rn32(a * C - Fraction(rn32(b * S))),
             "two roundings": rn32(Fraction(rn32(a * C)) - Fraction(rn32(b * S))),
             "fma on b*s": rn32(-b * S + Fraction(rn32(a * C)))}
    a, b = Fraction(1.25), Fraction(-0.8125)
    second = {"pinned": rn32(a * S + Fraction(rn32(b * C))),
              "two roundings": rn32(Fraction(rn32(a * S)) + Fraction(rn32(b * C))),
              "fma on b*c": rn32(b * C + Fraction(rn32(a * S)))}
    assert [f32bits(v) for v in first.values()] == [0x3D1D384A, 0x3D1D3850, 0x3D1D3856]
    assert [f32bits(v) for v in second.values()] == [0x3E55B236, 0x3E55B238, 0x3E55B23A]
    assert f32bits(z[0, 448]) == 0x3D1D384A
    assert f32bits(z[0, 451]) == 0x3E55B236


def test_rope_fma_form_exact_on_random_rows():
    # Every rotated value of random rows at random table positions against the
    # stated form evaluated exactly from the oracle's own pre-rotation y.
    rng = np.random.default_rng(23)
    tab = rope_table(131072)
    n = 48
    cs = tab[rng.integers(0, 131072, n)]
    y, z, _, _ = oracle.rows(rand_rows(n, 24), None, 1e-6, cs)
    diff_two = diff_other = 0
    for r in range(n):
        for i in range(32):
            a, b = Fraction(float(y[r, 448 + 2 * i])), Fraction(float(y[r, 449 + 2 * i]))
            c, s = Fraction(float(cs[r, i])), Fraction(float(cs[r, 32 + i]))
            bs, bc = Fraction(rn32(b * s)), Fraction(rn32(b * c))
            want_a, want_b = rn32(a * c - bs), rn32(a * s + bc)
            assert f32bits(z[r, 448 + 2 * i]) == f32bits(want_a), (r, i)
            assert f32bits(z[r, 449 + 2 * i]) == f32bits(want_b), (r, i)
            diff_two += rn32(Fraction(rn32(a * c)) - bs) != want_a
            diff_other += rn32(-b * s + Fraction(rn32(a * c))) != want_a
    assert diff_two > 0 and diff_other > 0
