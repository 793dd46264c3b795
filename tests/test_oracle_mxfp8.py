"""Pins of the oracle's MXFP8 norm-quant variant (residual add + Gemma RMSNorm +
32-element UE8M0 blocks + 128x4 swizzled scales): the page's helper rules by
their definitions, hand-computed swizzle offsets, closed forms for whole rows,
the odd-carry summation order, and error bounds."""
import numpy as np
import pytest

import oracle


def bf16(x):
    return oracle.f32_to_bf16(np.asarray(x, np.float32))


def f32(bits):
    return np.array([bits], np.uint32).view(np.float32)[0]


# ------------------------------------------------------------- UE8M0 ceil

def test_ue8m0_ceil_known_values():
    assert oracle.ue8m0_ceil_byte(1.0) == 127
    assert oracle.ue8m0_ceil_byte(2.0 ** -9) == 118
    assert oracle.ue8m0_ceil_byte(1.5) == 128
    assert oracle.ue8m0_ceil_byte(0.0) == 0
    assert oracle.ue8m0_ceil_byte(-3.0) == 0
    assert oracle.ue8m0_ceil_byte(f32(0x00400000)) == 0          # 2^-127, subnormal
    assert oracle.ue8m0_ceil_byte(f32(0x00400001)) == 1
    assert oracle.ue8m0_ceil_byte(f32(0x00000001)) == 0
    assert oracle.ue8m0_ceil_byte(2.0 ** 127) == 254
    assert oracle.ue8m0_ceil_byte(1.5 * 2.0 ** 127) == 254        # clamped


def test_ue8m0_ceil_is_the_rounded_up_exponent():
    rng = np.random.default_rng(61)
    bits = rng.integers(0x00400001, 0x7F000000, 20000, dtype=np.uint32)
    for v in bits.view(np.float32):
        b = oracle.ue8m0_ceil_byte(v)
        assert 1 <= b <= 254
        assert np.ldexp(1.0, b - 127) >= float(v)
        assert b == 1 or np.ldexp(1.0, b - 128) < float(v)


def test_ue8m0_inverse():
    for b in range(1, 254):
        assert oracle.ue8m0_inverse(b) == np.float32(2.0 ** (127 - b))
    assert oracle.ue8m0_inverse(0) == 0.0
    assert oracle.ue8m0_inverse(254) == 0.0       # 2^-127 is below the normal range: 0, as on the page
    assert oracle.ue8m0_inverse(255) == 0.0


def _byte_by_frexp(v):
    """The scale byte from frexp: v = f * 2^E with f in [0.5, 1), so the
    smallest power of two at or above v is 2^(E-1) when f is exactly 0.5 and
    2^E otherwise; its biased exponent, clamped to [0, 254], is the byte.
    +inf has no power of two above it and takes the cap, 254."""
    f, e = np.frexp(v.astype(np.float64))
    up = np.where(np.isinf(v), 254, e.astype(np.int64) - (f == 0.5) + 127)
    return np.where(v > 0, np.clip(up, 0, 254), 0).astype(np.uint8)


def test_ue8m0_byte_on_every_pattern():
    # Every positive finite fp32 pattern, +inf, both zeros and a stride of the
    # negative ones, against the frexp form of the definition.
    from test_oracle_formats import _over_chunks

    def check(start, stop):
        v = np.arange(start, stop, dtype=np.uint32).view(np.float32)
        return np.array_equal(oracle.ue8m0_ceil_bytes(v), _byte_by_frexp(v))
    assert _over_chunks(check, 0, 0x7F800001) == []
    neg = (np.arange(0x80000000, 0xFF800001, 4093, dtype=np.uint64)).astype(np.uint32).view(np.float32)
    assert not oracle.ue8m0_ceil_bytes(neg).any()


# ------------------------------------------------------------- swizzle

def test_swizzled_offsets_by_hand():
    pc = 8
    cases = {(0, 0): 0, (0, 1): 1, (0, 3): 3, (0, 4): 512, (0, 7): 515, (1, 0): 16,
             (31, 0): 496, (32, 0): 4, (96, 0): 12, (127, 3): 511, (128, 0): 128 * pc,
             (130, 5): 128 * pc + 512 + 1 + 32}
    for (r, c), want in cases.items():
        assert oracle.mxfp8_scale_offset(r, c, pc) == want, (r, c)


def test_swizzle_is_a_bijection_per_tile():
    pc = 12
    offs = sorted(oracle.mxfp8_scale_offset(r, c, pc) for r in range(256) for c in range(pc))
    assert offs == list(range(256 * pc))


# ------------------------------------------------------------- whole rows

def test_constant_power_of_two_rows_closed_form():
    # x = 2^k at eps = 0 with gamma = 0: normed = 1 exactly, amax = 1,
    # v = RN(1/448) in [2^-9, 2^-8) with a non-zero mantissa -> byte 119,
    # inverse 2^8 -> 256 -> code 0x78.
    m, hidden = 5, 256
    for k in (-6, 0, 9):
        x = bf16(np.full((m, hidden), 2.0 ** k))
        codes, scales, _ = oracle.mxfp8_norm_quant(x, bf16(np.zeros(hidden)), 0.0)
        assert np.all(codes == 0x78)
        pc = hidden // 32
        valid = np.zeros(scales.size, bool)
        for r in range(m):
            for c in range(pc):
                valid[oracle.mxfp8_scale_offset(r, c, pc)] = True
        assert np.all(scales[valid] == 119)
        assert np.all(scales[~valid] == 0)                  # padding rows 5..127 zeroed


def test_gemma_weight_and_residual_add():
    rng = np.random.default_rng(62)
    hidden = 384
    g = bf16(0.25 * rng.standard_normal(hidden))
    x = bf16(np.ones((2, hidden)))
    r = np.zeros((2, hidden), np.uint16)
    r[1, :] = bf16(np.full(hidden, 2.0 ** -8))     # 1 + 2^-8 ties to 1.0 in bf16
    codes, scales, pre = oracle.mxfp8_norm_quant(x, g, 0.0, residual=r)
    assert np.all(pre == 0x3F80)
    # normed = bf16(1 * (g + 1)); its codes must dequantize within the E4M3 bound
    normed = oracle.bf16_to_f32(bf16(oracle.bf16_to_f32(g).astype(np.float32) + np.float32(1.0)))
    pc = hidden // 32
    for row in range(2):
        for c in range(pc):
            b = scales[oracle.mxfp8_scale_offset(row, c, pc)]
            deq = oracle.e4m3_to_f64(codes[row, 32 * c:32 * c + 32]) * 2.0 ** (int(b) - 127)
            want = normed[32 * c:32 * c + 32].astype(np.float64)
            assert np.all(np.abs(deq - want) <= 2.0 ** -4 * np.abs(want) + 2.0 ** (int(b) - 137))
    r2 = np.zeros((1, hidden), np.uint16)
    r2[0, :] = bf16(np.full(hidden, 3 * 2.0 ** -8))
    _, _, pre2 = oracle.mxfp8_norm_quant(x[:1], g, 0.0, residual=r2)
    assert np.all(pre2 == 0x3F82)                   # 1 + 3*2^-8 ties up to the even 0x3F82


def test_bf16_rounding_before_quant_decides_a_tie():
    # One row of ones at eps = 0 (inv = 1), hidden 128.  gamma[0] = 0.75 gives
    # normed 1.75, the block amax: v = RN(1.75 * RN(1/448)) = 2^-8 exactly
    # (RN(1/448) is 1/448 * (1 + 4.5e-8) and 1.75 times it rounds back to
    # 2^-8), so byte 119 and inverse 2^8.  gamma[1] = 0.1865234375 gives
    # g + 1 = 1.1865234375, whose bf16 is 1.1875: 1.1875 * 256 = 304 is the tie
    # between 288 (mantissa 1) and 320 (mantissa 2), so code 0x7a; without the
    # bf16 rounding, 303.75 would round to 288, code 0x79.
    g = np.zeros(128, np.float32)
    g[0] = 0.75
    g[1] = 0.1865234375
    codes, scales, _ = oracle.mxfp8_norm_quant(bf16(np.ones((1, 128))), bf16(g), 0.0)
    assert codes[0, 0] == 0x7E and codes[0, 1] == 0x7A
    assert np.all(codes[0, 2:] == 0x78)
    assert all(scales[oracle.mxfp8_scale_offset(0, c, 4)] == 119 for c in range(4))


def _sumsq_n(x):
    buf = np.ascontiguousarray(bf16(x))       # keep the buffer alive across the call
    return oracle.lib().orc_sum_squares_n(buf.ctypes.data, buf.size)


def test_sum_of_squares_carries_the_odd_element():
    # hidden 1536 = 192 chunks = three aligned groups of 64 chunks.  With
    # 2^24 in group 0 and 1 in groups 1 and 2: ((G0 + G1) + G2) = 2^24 (each
    # + 1 ties to even), while G0 + (G1 + G2) would be 2^24 + 2.
    x = np.zeros(1536, np.float32)
    x[0] = 4096.0
    x[64 * 8] = 1.0
    x[128 * 8] = 1.0
    assert _sumsq_n(x) == 2.0 ** 24
    # the first six levels stay inside each aligned group of 64 chunks
    y = np.zeros(1536, np.float32)
    y[0] = 4096.0
    y[8] = y[16] = y[24] = 1.0
    assert _sumsq_n(y) == 2.0 ** 24 + 2


@pytest.mark.parametrize("hidden", [128, 512, 1536, 4096, 7168])
def test_random_rows_against_float64(hidden):
    rng = np.random.default_rng(hidden)
    m = 7
    x = bf16(rng.standard_normal((m, hidden)))
    res = bf16(0.5 * rng.standard_normal((m, hidden)))
    g = bf16(0.1 * rng.standard_normal(hidden))
    eps = 1e-6
    codes, scales, pre = oracle.mxfp8_norm_quant(x, g, eps, residual=res)
    # prenorm is the bf16 of the fp32 sum
    xs = oracle.bf16_to_f32(x).astype(np.float32) + oracle.bf16_to_f32(res).astype(np.float32)
    assert np.array_equal(pre, bf16(xs))
    p = oracle.bf16_to_f32(pre).astype(np.float64)
    ideal = p / np.sqrt((p ** 2).mean(axis=1, keepdims=True) + np.float64(np.float32(eps))) * \
        (oracle.bf16_to_f32(g).astype(np.float64) + 1.0)
    pc = hidden // 32
    for r in range(m):
        for c in range(pc):
            b = int(scales[oracle.mxfp8_scale_offset(r, c, pc)])
            blk = ideal[r, 32 * c:32 * c + 32]
            deq = oracle.e4m3_to_f64(codes[r, 32 * c:32 * c + 32]) * 2.0 ** (b - 127)
            # bf16 rounding (2^-9 relative) plus E4M3 rounding (2^-4) plus fp32 noise
            assert np.all(np.abs(deq - blk) <= (2.0 ** -4 + 2.0 ** -8) * np.abs(blk) + 2.0 ** (b - 136))
            assert 448.0 * 2.0 ** (b - 127) >= np.abs(blk).max() * (1 - 2.0 ** -7)


def test_hidden_must_be_a_multiple_of_128():
    with pytest.raises(ValueError):
        oracle.mxfp8_norm_quant(np.zeros((1, 96), np.uint16), np.zeros(96, np.uint16), 1e-6)


def test_odd_carry_tree_equals_the_zero_padded_tree():
    # The summation order (chunks of 8 left to right, adjacent pairs level by
    # level, an odd last value carried up) gives the same bits as the same tree
    # over the row padded with zero chunks to a power-of-two count, because a
    # carried x and x + 0 are the same number.  A kernel that splits rows into
    # whole groups of 64 chunks and pads the last group relies on this.
    rng = np.random.default_rng(71)
    for n in (128, 384, 640, 1152, 3200, 8704, 12288, 16256):
        x = bf16(rng.standard_normal(n) * np.exp(rng.uniform(-8, 8, n)))
        width = 1 << int(np.ceil(np.log2(n)))
        padded = np.concatenate([x, np.zeros(width - n, np.uint16)])
        a = oracle.lib().orc_sum_squares_n(np.ascontiguousarray(x).ctypes.data, n)
        b = oracle.lib().orc_sum_squares_n(np.ascontiguousarray(padded).ctypes.data, width)
        assert np.float32(a).view(np.uint32) == np.float32(b).view(np.uint32), n


# ------------------------------------------------------------- exact arithmetic
#
# tests/mx_exact.py evaluates readings M1-M6 in exact rational arithmetic with
# one rounding per stated step, independently of the oracle.  The oracle must
# match it code for code and byte for byte; the cases below are chosen so that
# the alternative readings it can also evaluate (eps outside the root, the norm
# reading the binary32 sum instead of its bf16 rounding, the Gemma weight
# applied before inv) give different codes.

from fractions import Fraction  # noqa: E402

import mx_exact as X  # noqa: E402


def _bits(vals):
    """bf16 bit patterns of values that are bf16 numbers (checked)."""
    f = np.array([float(v) for v in vals], np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), f)
    return b


def _oracle_row(x, gamma, eps, residual=None):
    hidden = len(x)
    codes, scales, _ = oracle.mxfp8_norm_quant(_bits(x)[None, :], _bits(gamma), eps,
                                               residual=None if residual is None else _bits(residual)[None, :])
    pc = hidden // 32
    return [int(c) for c in codes[0]], [int(scales[oracle.mxfp8_scale_offset(0, c, pc)]) for c in range(pc)]


def test_exact_helper_known_values():
    assert X.sqrt_rn32(Fraction(9)) == 3
    assert np.float32(float(X.sqrt_rn32(Fraction(2)))).view(np.uint32) == 0x3FB504F3
    assert X.sqrt_rn32(Fraction(1, 4)) == Fraction(1, 2)
    assert X.bf16(1 + Fraction(1, 256)) == 1                      # tie to the even significand
    assert X.bf16(1 + Fraction(3, 256)) == 1 + Fraction(1, 64)
    assert X.rn32(Fraction(1, 3)) == Fraction(11184811, 2 ** 25)
    assert [X.e4m3(v) for v in (448, 304, 288, Fraction(1, 512), Fraction(3, 1024), Fraction(1, 1024), -1)] == \
        [0x7E, 0x7A, 0x79, 0x01, 0x02, 0x00, 0xB8]
    assert X.scale_byte(Fraction(1, 256)) == 119 and X.scale_byte(Fraction(1, 256) * (1 + Fraction(1, 2 ** 23))) == 120
    assert X.scale_byte(0) == 0 and X.scale_byte(Fraction(1, 2 ** 140)) == 0


def test_eps_inside_the_root():
    # x = 2 everywhere, gamma = 0, eps = 5: S = 128 * 4, mean 4, RN(4 + 5) = 9,
    # root 3, inv = RN(1/3), t = RN(2 * inv) = 0.666666686..., whose bf16 is
    # 0.66796875: v = RN(0.66796875 * RN(1/448)) lies in (2^-10, 2^-9], byte
    # 118, inverse 2^9, 342 -> 352, code 0x7b.  With eps outside the root:
    # inv = RN(1/7), n = bf16(2/7) = 0.28515625, byte 117, 292 -> 288, code 0x79.
    x, g = [2] * 128, [0] * 128
    codes, bytes_ = _oracle_row(x, g, 5.0)
    assert codes == [0x7B] * 128 and bytes_ == [118] * 4
    assert (codes, bytes_) == X.row(x, g, 5.0)
    assert X.row(x, g, 5.0, eps_outside=True) == ([0x79] * 128, [117] * 4)


def _residual_case(seed, hidden=128, k=8):
    # k non-zero elements (integers 1..3) with residuals of +-1 or 3 / 256, so
    # that x + residual is not always a bf16 number and the sum of squares stays
    # exact in binary32; weights in steps of 1/64.
    rng = np.random.default_rng(seed)
    x = [Fraction(0)] * hidden
    r = [Fraction(0)] * hidden
    for j in rng.choice(hidden, k, replace=False):
        x[j] = Fraction(int(rng.integers(1, 4)))
        r[j] = Fraction(int(rng.choice([-3, -1, 1, 3])), 256)
    g = [Fraction(int(v), 64) for v in rng.integers(-16, 17, hidden)]
    return x, r, g


def test_norm_reads_the_bf16_residual_sum():
    # Seeds where the readings part: at 12 the binary32 sum read in both the
    # sum of squares and the scaling moves block 2's byte (119 -> 120); at 40
    # it moves block 2's byte (122 -> 121) also when only the scaling reads it.
    x, r, g = _residual_case(12)
    got = _oracle_row(x, g, 0.0, residual=r)
    assert got == X.row(x, g, 0.0, residual=r)
    alt = X.row(x, g, 0.0, residual=r, fp32_sum=True)
    assert got[1][2] == 119 and alt[1][2] == 120
    x, r, g = _residual_case(40)
    got = _oracle_row(x, g, 0.0, residual=r)
    assert got == X.row(x, g, 0.0, residual=r)
    assert got[1][2] == 122
    for alt in (X.row(x, g, 0.0, residual=r, fp32_sum=True), X.row(x, g, 0.0, residual=r, fp32_scaled=True)):
        assert alt[1][2] == 121 and alt[0] != got[0]


def test_gemma_weight_applied_after_inv():
    # x = 7 everywhere at eps = 0: inv = RN(1/7) and RN(7 * inv) = 1, so n is
    # the bf16 of (gamma + 1); with the weight first, RN(RN(7 * (gamma + 1)) * inv)
    # moves some of them by an ulp, and at this seed one across an E4M3 midpoint.
    rng = np.random.default_rng(0)
    g = [X.bf16(Fraction(int(v), 512)) for v in rng.integers(-200, 201, 128)]
    x = [7] * 128
    got = _oracle_row(x, g, 0.0)
    assert got == X.row(x, g, 0.0)
    assert X.row(x, g, 0.0, weight_first=True)[0] != got[0]


@pytest.mark.parametrize("hidden,with_residual,eps", [(128, False, 0.0), (512, True, 1e-6), (1536, True, 0.0),
                                                     (7168, False, 1e-6)])
def test_dyadic_rows_code_for_code(hidden, with_residual, eps):
    # Quarter-integer inputs keep every sum of squares exact (and every
    # residual sum a bf16 number), so the whole row is fixed by the readings.
    rng = np.random.default_rng(hidden)
    x = [Fraction(int(v), 4) for v in rng.integers(-16, 17, hidden)]
    x = [v if v != 0 else Fraction(1, 4) for v in x]
    r = [Fraction(int(v), 4) for v in rng.integers(-8, 9, hidden)] if with_residual else None
    if r is not None:
        r = [b if a + b != 0 else b + Fraction(1, 4) for a, b in zip(x, r)]
    g = [X.bf16(Fraction(int(v), 256)) for v in rng.integers(-60, 61, hidden)]
    eps32 = float(np.float32(eps))
    assert _oracle_row(x, g, eps32, residual=r) == X.row(x, g, Fraction(eps32), residual=r)
