"""Nonlinear approximation unit: 2^v, e^x, SoftPlus and SiLU in Q.16 integers.

[FM] "What carries the argument": the nonlinearities reduce to an 8-segment
first-order linear approximation of 2^v, with e^x = 2^(x log2 e) and the
symmetry SoftPlus(x) = x + SoftPlus(-x).  [FM] minor comment on Section
III-B.2: Eq. (5) approximates SoftPlus(x) by e^x, the domain x <= 0 being
implied by the symmetry argument.  [FMV] supporting citations: [15] supplies
the shift-based exponential used for e^dt in the SSM block, [16] the symmetry
that lets SoftPlus reuse the exponential unit.

Readings (the pages give the form, not the coefficients or widths):
* Q.16: int32 with 16 fraction bits, for inputs and outputs.
* The 8 segments split each octave [n, n+1) of v into eighths; segment i is
  the chord between 2^(i/8) and 2^((i+1)/8), the table holding
  Y[i] = rint(2^(i/8) * 2^30) for i = 0..8.  Inside a segment the remaining
  13 fraction bits r interpolate: m = Y[i] + rshr((Y[i+1]-Y[i]) * r, 13), and
  the integer part n becomes the shift: 2^v ~ rshr(m, 14 - n) in Q.16.
* log2(e) is the integer LOG2E_Q30 = rint(log2(e) * 2^30).
* The exponential is only ever needed for arguments <= 0 (decay e^(dt*A),
  SoftPlus through the symmetry, SiLU through the symmetry below), where
  e^x lies in [0, 1] and its Q.16 value fits in [0, 2^16].
* SoftPlus(x) = e^(-|x|) + max(x, 0): Eq. (5) on x <= 0, the symmetry for x > 0.
* SiLU, which the pages' approximation does not cover, uses the same unit
  and the same symmetry, SiLU(x) = x + SiLU(-x): for x <= 0,
  sigma(x) = E / (1 + E) with E = e^x, computed as floor(E*2^16 / (2^16 + E)),
  and SiLU(x) = rshr(x * sigma, 16).
"""
import numpy as np

from .fixedpoint import I32_MAX, I32_MIN, rshr, sat32


def _exp2_table():
    # rint(2^(i/8) * 2^30) from the defining real numbers (float64 is ample: no
    # value lies within 1e-6 of a rounding boundary; the pins recompute these
    # with exact integer roots)
    return np.array([int(np.rint(2.0 ** (i / 8.0) * 2.0 ** 30)) for i in range(9)],
                    dtype=np.int64)


EXP2_TABLE_Q30 = _exp2_table()
LOG2E_Q30 = int(np.rint(np.log2(np.e) * 2.0 ** 30))


def exp2_q16(v, table=None):
    """2^(v / 2^16) in Q.16 for Q.16 integers v <= 0 (result in [0, 2^16]).

    ``table``: nine Q.30 knots in place of EXP2_TABLE_Q30 (alternative fits of
    the same piecewise-linear form)."""
    tab = EXP2_TABLE_Q30 if table is None else np.asarray(table, dtype=np.int64)
    v = np.asarray(v, dtype=np.int64)
    assert np.all(v <= 0), "the exponential unit is used for arguments <= 0 only"
    # below -32 the result is 0 whatever the segment (the shift exceeds 45 bits)
    v = np.maximum(v, -(32 << 16))
    n = v >> 16                       # integer part (floor)
    f = v - (n << 16)                 # fraction in [0, 2^16)
    i = f >> 13                       # segment 0..7
    r = f & 0x1FFF                    # position inside the segment, 13 bits
    y0 = tab[i]
    y1 = tab[i + 1]
    m = y0 + rshr((y1 - y0) * r, 13)  # Q.30 mantissa in [2^30, 2^31]
    return rshr(m, 14 - n)


def exp_q16(x, table=None):
    """e^(x / 2^16) in Q.16 for Q.16 integers x in [-2^31, 0]."""
    x = np.asarray(x, dtype=np.int64)
    assert np.all((x <= 0) & (x >= I32_MIN))
    return exp2_q16(rshr(x * LOG2E_Q30, 30), table)


def softplus_q16(x, table=None):
    """SoftPlus in Q.16: e^(-|x|) + max(x, 0), saturated to int32."""
    x = np.asarray(x, dtype=np.int64)
    assert np.all((x >= I32_MIN) & (x <= I32_MAX))
    return sat32(exp_q16(-np.abs(x), table) + np.maximum(x, 0))


def silu_q16(x, table=None):
    """SiLU in Q.16 through the exponential unit and SiLU(x) = x + SiLU(-x)."""
    x = np.asarray(x, dtype=np.int64)
    assert np.all((x >= I32_MIN) & (x <= I32_MAX))
    xn = -np.abs(x)                               # <= 0
    e = exp_q16(xn, table)                        # e^xn in [0, 2^16] (chord table)
    sig = (e << 16) // ((1 << 16) + e)            # sigma(xn) in Q.16, floor
    sn = rshr(xn * sig, 16)                       # SiLU(xn)
    return np.where(x > 0, x + sn, sn)
