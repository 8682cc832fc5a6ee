"""Pins of the oracle's FP32 scale rule against exact rational arithmetic (CPU).

The rule (the "DeepSeek-V3: the recipe, and the interconnect that shaped it"
page, section "FP8: the other half of the byte reduction"; the book's chapter
16 "Scaling a group" and "Online scales"): per tile, scale = amax / 448 held
in FP32, and each value is divided by the scale and cast to E4M3.  Reading:
both steps are IEEE FP32 operations rounded to nearest even, then the cast
rounds to nearest even, saturating, so the code is E4M3(fl32(x / fl32(amax /
448))) -- two roundings of the quotient, in that order.

The expected values here come from Python's exact ``fractions.Fraction``
arithmetic and a rounding routine written from the IEEE definition (round the
exact rational to the nearest value with 24 significant bits, ties to even),
not from numpy's FP32 division.  The cases are chosen where plausible wrong
oracles differ from the rule:

* a scale that is not a power of two (amax = 300), where x * (1/s) and x / s
  can differ;
* values where fl32(x * fl32(1 / s)) and fl32(x / s) give different E4M3
  codes (a reciprocal-multiply oracle fails them);
* values where fl32(x / s) lands exactly on an E4M3 rounding midpoint although
  x / s itself does not, so the two-step reading ties to the even code while a
  single rounding of the exact quotient goes the other way (an oracle that
  rounds once from float64 fails them).
"""

from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import fp8, quant


def _ilog2(a):
    """floor(log2(a)) of a positive Fraction, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fr(2) ** e > a:
        e -= 1
    elif Fr(2) ** (e + 1) <= a:
        e += 1
    return e


def _round_to_grid(a, step):
    """a / step rounded to the nearest integer, ties to even, times step."""
    q = a / step
    n = q.numerator // q.denominator
    r = q - n
    if r > Fr(1, 2) or (r == Fr(1, 2) and n % 2 == 1):
        n += 1
    return n * step


def rn_f32(x):
    """Exact rational x rounded to the nearest FP32 value (ties to even)."""
    if x == 0:
        return Fr(0)
    a = abs(x)
    e = max(_ilog2(a), -126)
    v = _round_to_grid(a, Fr(2) ** (e - 23))
    return v if x > 0 else -v


def rn_e4m3(x):
    """Exact rational x to the nearest E4M3 value (ties to even, subnormals
    kept, saturating at 448)."""
    if x == 0:
        return Fr(0)
    a = abs(x)
    e = max(_ilog2(a), -6)
    v = min(_round_to_grid(a, Fr(2) ** (e - 3)), Fr(448))
    return v if x > 0 else -v


def is_e4m3_midpoint(v):
    a = abs(v)
    if a == 0 or a >= 448:
        return False
    e = max(_ilog2(a), -6)
    q = a / Fr(2) ** (e - 4)          # in units of half a step
    return q.denominator == 1 and q.numerator % 2 == 1


def bf16_values(lo, hi):
    """All positive BF16 values in [lo, hi)."""
    out = []
    for e in range(-20, 20):
        for m in range(128):
            v = Fr(128 + m, 128) * Fr(2) ** e
            if lo <= v < hi:
                out.append(v)
    return out


def oracle_code_value(amax, x):
    """The oracle's decoded code of x in a 1x128 tile whose max-abs is amax."""
    t = np.zeros((1, 128), np.float32)
    t[0, 0] = float(amax)
    t[0, 1] = float(x)
    q, s = quant.quant_1x128(t)
    return Fr(float(fp8.e4m3_decode(q[0, 1]))), Fr(float(s[0, 0]))


def test_scale_of_a_non_power_of_two_amax():
    s = rn_f32(Fr(300) / 448)
    assert s != Fr(300, 448)                       # 75/112 is not an FP32 value
    _, got = oracle_code_value(300, 0)
    assert got == s


def _cases(amaxes):
    recip, single = [], []
    for amax in amaxes:
        s = rn_f32(amax / 448)
        inv = rn_f32(1 / s)
        for x in bf16_values(amax / 64, amax):
            two_step = rn_e4m3(rn_f32(x / s))
            if rn_e4m3(rn_f32(x * inv)) != two_step:
                recip.append((amax, x, two_step))
            if is_e4m3_midpoint(rn_f32(x / s)) and x / s != rn_f32(x / s) and rn_e4m3(x / s) != two_step:
                single.append((amax, x, two_step))
    return recip, single


@pytest.fixture(scope="module")
def cases():
    # every BF16 amax in [256, 320): the scale's FP32 rounding varies over them
    return _cases(bf16_values(256, 320))


def test_reciprocal_multiply_differs(cases):
    """Codes where x * fl32(1/s) gives another code than x / s: the oracle
    takes the quotient."""
    recip, _ = cases
    assert len(recip) >= 3, len(recip)
    for amax, x, want in recip:
        got, _ = oracle_code_value(amax, x)
        assert got == want, (float(amax), float(x), float(got), float(want))
        got_neg, _ = oracle_code_value(amax, -x)
        assert got_neg == -want


def test_double_rounding_on_a_midpoint(cases):
    """fl32(x / s) is exactly an E4M3 midpoint while x / s is not: the
    two-step rule ties to the even code, a single rounding would not."""
    _, single = cases
    assert len(single) >= 1, len(single)
    for amax, x, want in single:
        got, _ = oracle_code_value(amax, x)
        assert got == want, (float(amax), float(x), float(got), float(want))
        # the two readings give the two neighbours of the midpoint
        s = rn_f32(amax / 448)
        mid = rn_f32(x / s)
        other = rn_e4m3(x / s)
        assert other != want and abs(want - mid) == abs(mid - other)


def test_rounding_helpers_on_hand_values():
    """The exact helpers against values worked by hand."""
    assert rn_f32(Fr(1, 3)) == Fr(11184811, 33554432)          # 0x3EAAAAAB
    assert rn_f32(Fr(300, 448)) == Fr(11234743, 16777216)      # 0x3F2B6DB7
    assert rn_e4m3(Fr(17, 16)) == Fr(1)          # tie between 1 and 1.125: even (1.000)
    assert rn_e4m3(Fr(19, 16)) == Fr(5, 4)       # tie between 1.125 and 1.25: even (1.010)
    assert rn_e4m3(Fr(500)) == 448               # saturates
    assert rn_e4m3(Fr(3, 2048)) == Fr(1, 512)    # 0.75 * 2^-9 rounds up to the smallest subnormal
    assert rn_e4m3(Fr(1, 1024)) == 0             # 0.5 * 2^-9: tie between 0 and 2^-9, even is 0
    assert rn_e4m3(Fr(3, 1024)) == Fr(1, 256)    # 1.5 * 2^-9: tie between 1 and 2 steps, even is 2
    assert is_e4m3_midpoint(Fr(17, 16)) and not is_e4m3_midpoint(Fr(9, 8))
