"""The FP32 division sequence of the expert GEMM's requantisation, checked in
exact rational arithmetic (CPU).

The kernels divide each element of a 1x128 tile of h by the tile's scale s
(fl32(x / s) before the E4M3 cast, the same correctly rounded quotient the
activation quantiser takes).  Instead of a full IEEE division per element
they compute r = fl32(1 / s) once and per element
    q0 = fl32(x r);  q1 = fma(fma(-s, q0, x), r, q0);  q = fma(fma(-s, q1, x), r, q1)
with FMAs rounding once (IEEE).  Markstein's theorem makes q the correctly
rounded quotient once q1 is within an ulp of x / s (then the second remainder
is exact).  This test replays the sequence with exact rationals rounded to
FP32 at every step and compares with the correctly rounded x / s, on random
operands, on quotients next to FP32 rounding midpoints, and on divisors
whose significand is all ones.
"""

import random
from fractions import Fraction as Fr

from tests.test_oracle_quant_rule import rn_f32


def _f32(rng, lo=-40, hi=40):
    return Fr(rng.randint(1 << 23, (1 << 24) - 1)) * Fr(2) ** (rng.randint(lo, hi) - 23)


def _sequence(x, s):
    r = rn_f32(1 / s)
    q0 = rn_f32(x * r)
    q1 = rn_f32(q0 + rn_f32(x - s * q0) * r)
    e1 = x - s * q1
    assert rn_f32(e1) == e1, "second remainder not exact"
    return rn_f32(q1 + e1 * r)


def test_division_sequence_is_correctly_rounded():
    rng = random.Random(7)
    cases = [(_f32(rng), _f32(rng)) for _ in range(6000)]
    for _ in range(6000):                      # quotients at an FP32 rounding midpoint
        s, q = _f32(rng, -10, 10), _f32(rng, -10, 10)
        e = q.numerator.bit_length() - q.denominator.bit_length()
        cases.append((rn_f32((q + Fr(2) ** (e - 25)) * s), s))
    for _ in range(2000):                      # divisors with an all-ones significand
        cases.append((_f32(rng), Fr((1 << 24) - 1) * Fr(2) ** rng.randint(-30, 0)))
    for x, s in cases:
        assert _sequence(x, s) == rn_f32(x / s), (float(x), float(s))
        assert _sequence(-x, s) == -rn_f32(x / s)
