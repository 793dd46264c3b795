"""An exact-arithmetic evaluation of the MXFP8 norm-quant rules (readings
M1-M6 of the vLLM MiniMax page's _LamportGemmaRMSNormMxfp8Kernel, restated),
written independently of the oracle: every value is a Fraction, every step
rounds once, to binary32 or bf16 (round to nearest, ties to even) or to the
nearest E4M3 value, exactly where the readings say.  It serves the CPU pins:
the oracle must reproduce it code for code, and the alternative readings it
can also evaluate must not.

It covers rows whose sum of squares is exact in binary32 (the callers check
`sum_is_exact`): then the summation order, which other pins fix, cannot
matter."""
import math
from fractions import Fraction


def round_sig(x, bits, emin=-126, emax=127):
    """x rounded to `bits` significant bits (ties to even), with the fixed
    quantum of 2^(emin - bits + 1) below 2^emin; None past the largest finite
    value (the callers stay in range)."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    neg, m = x < 0, abs(x)
    e = m.numerator.bit_length() - m.denominator.bit_length()
    if Fraction(2) ** e > m:
        e -= 1
    elif Fraction(2) ** (e + 1) <= m:
        e += 1
    quantum = Fraction(2) ** (max(e, emin) - bits + 1)
    v = round(m / quantum) * quantum             # Fraction.__round__ ties to even
    if v >= Fraction(2) ** (emax + 1):
        return None
    return -v if neg else v


def rn32(x):
    return round_sig(x, 24)


def bf16(x):
    return round_sig(x, 8)


def sqrt_rn32(v):
    """The binary32 value nearest to sqrt(v), v > 0 rational: the candidate
    whose rounding interval [r - u/2, r + u/2] holds sqrt(v), compared in
    squares."""
    v = Fraction(v)
    r0 = rn32(Fraction(math.sqrt(float(v))))
    e = r0.numerator.bit_length() - r0.denominator.bit_length()
    if Fraction(2) ** e > r0:
        e -= 1
    for r in (r0, r0 - Fraction(2) ** (e - 23), r0 + Fraction(2) ** (e - 23),
              r0 - Fraction(2) ** (e - 24), r0 + Fraction(2) ** (e - 24)):
        if r <= 0 or rn32(r) != r:
            continue
        re = r.numerator.bit_length() - r.denominator.bit_length()
        if Fraction(2) ** re > r:
            re -= 1
        ulp_up = Fraction(2) ** (re - 23)
        ulp_down = ulp_up / 2 if r == Fraction(2) ** re else ulp_up
        lo, hi = r - ulp_down / 2, r + ulp_up / 2
        if lo * lo < v < hi * hi:
            return r
        if v in (lo * lo, hi * hi):                 # a tie: the even significand
            if (r / ulp_up).numerator % 2 == 0:
                return r
    raise AssertionError("no binary32 square root found for %s" % v)


def _e4m3_values():
    out = []
    for code in range(0x7F):                        # 0x7F is NaN
        ex, man = code >> 3, code & 7
        val = Fraction(man, 8) * Fraction(2) ** -6 if ex == 0 else (1 + Fraction(man, 8)) * Fraction(2) ** (ex - 7)
        out.append((val, code))
    return out


E4M3 = _e4m3_values()


def e4m3(x):
    """The E4M3 code nearest to x (|x| <= 448), ties to the even code."""
    x = Fraction(x)
    sign = 0x80 if x < 0 else 0x00
    a = abs(x)
    assert a <= 448
    best = min(E4M3, key=lambda vc: (abs(vc[0] - a), vc[1] & 1))
    return sign | best[1]


INV448 = rn32(Fraction(1, 448))


def scale_byte(v):
    """The least b >= 0 with v <= 2^(b - 127), at most 254; 0 for v <= 0."""
    if v <= 0:
        return 0
    b = 0
    while b < 254 and v > Fraction(2) ** (b - 127):
        b += 1
    return b


def sum_is_exact(p):
    """Every partial sum of squares of p exact in binary32 (then any order
    gives the exact sum)."""
    s = Fraction(0)
    for v in p:
        s += Fraction(v) ** 2
        if rn32(s) != s:
            return False
    return True


def row(x, gamma, eps, residual=None, eps_outside=False, fp32_sum=False, fp32_scaled=False,
        weight_first=False):
    """Codes [hidden] and scale bytes [hidden / 32] of one row.  x, residual,
    gamma: sequences of the bf16 values (as floats or Fractions); eps a
    binary32 value.  The flags evaluate alternative readings instead of the
    stated ones: eps added outside the root, the norm reading the binary32 sum
    instead of its bf16 rounding (fp32_sum: in the sum of squares and in the
    scaling; fp32_scaled: in the scaling only), and (p * (gamma + 1)) * inv."""
    hidden = len(x)
    if residual is None:
        s32 = [Fraction(v) for v in x]
        p = list(s32)
    else:
        s32 = [rn32(Fraction(a) + Fraction(b)) for a, b in zip(x, residual)]
        p = [bf16(v) for v in s32]                                   # M1: the residual output
    normsrc = s32 if fp32_sum else p
    assert sum_is_exact(normsrc)
    S = sum(Fraction(v) ** 2 for v in normsrc)
    mean = rn32(S / hidden)
    eps = Fraction(eps)
    if eps_outside:
        inv = rn32(1 / rn32(sqrt_rn32(mean) + eps))
    else:
        inv = rn32(1 / sqrt_rn32(rn32(mean + eps)))                  # M3
    n = []
    for v, g in zip(s32 if fp32_scaled else normsrc, gamma):
        g1 = rn32(Fraction(g) + 1)
        if weight_first:
            n.append(bf16(rn32(rn32(v * g1) * inv)))
        else:
            n.append(bf16(rn32(rn32(v * inv) * g1)))                 # M4
    codes, bytes_ = [], []
    for b in range(hidden // 32):
        blk = n[32 * b:32 * b + 32]
        amax = max(abs(v) for v in blk)
        byte = scale_byte(rn32(amax * INV448))                       # M5
        inverse = Fraction(2) ** (127 - byte) if 1 <= byte <= 253 else Fraction(0)
        bytes_.append(byte)
        codes += [e4m3(max(min(v * inverse, 448), -448)) for v in blk]   # M6
    return codes, bytes_
