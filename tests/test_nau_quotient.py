"""Host-side check of the numerical argument behind the device form of the 2^v
unit's SiLU quotient (no GPU): sigma = floor(E*2^16 / (2^16 + E)) is taken as
floor(E * r1 + 2^-20), r1 being one Newton step on a float64 reciprocal of
b = 1 + E*2^-16.  For every E the unit produces (0 .. 2^16) and a reciprocal
whose relative error is anywhere in [-2^-18, 2^-18] (the hardware's is near
2^-23), each float64 operation rounded to nearest as the device rounds it,
the result must equal the integer quotient.  The error enters monotonically,
so the two ends of the interval and the exact reciprocal cover it."""
from fractions import Fraction

import pytest

TINY = 2.0 ** -20


def _fma(a, b, c):
    return float(Fraction(a) * Fraction(b) + Fraction(c))  # one rounding


def _sigma(e, eps):
    b = _fma(e, 2.0 ** -16, 1.0)
    r0 = float(Fraction(1) / Fraction(b) * (1 + Fraction(eps)))
    r1 = _fma(r0, _fma(-b, r0, 1.0), r0)
    return int(_fma(e, r1, TINY) // 1)


@pytest.mark.parametrize("eps", [-2.0 ** -18, 0.0, 2.0 ** -18])
def test_silu_quotient_every_e(eps):
    bad = [e for e in range(0, (1 << 16) + 1)
           if _sigma(float(e), eps) != (e << 16) // ((1 << 16) + e)]
    assert not bad, bad[:10]


def test_silu_quotient_needs_the_newton_step():
    # without the refinement a reciprocal error of 2^-18 gives wrong quotients:
    # the check above is not vacuous
    def raw(e, eps):
        b = _fma(e, 2.0 ** -16, 1.0)
        r0 = float(Fraction(1) / Fraction(b) * (1 + Fraction(eps)))
        return int(_fma(e, r0, TINY) // 1)
    assert any(raw(float(e), 2.0 ** -18) != (e << 16) // ((1 << 16) + e) for e in range(1 << 16))
