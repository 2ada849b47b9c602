"""Fixed-point primitives: saturation, rounding shifts, power-of-two exponents.

[FM] "What carries the argument": the SSM block and the convolution use
power-of-two scale factors 2^p so that every rescaling is a shift.  The pages
give neither the bit widths nor the rounding; the readings taken here:

* reading: int8 codes are symmetric, clamped to [-127, 127]; accumulators and
  fixed-point values are int32, saturated to [-2^31, 2^31-1].
* reading: a right shift by s rounds half up, floor(v / 2^s + 1/2); a negative
  s is an exact left shift.
* reading: the exponent p of a tensor with absolute maximum a is the largest
  integer with a * 2^p <= 127 (no value clips), limited to [PMIN, PMAX].
"""
import numpy as np

I32_MIN = -(1 << 31)
I32_MAX = (1 << 31) - 1
PMIN = -24
PMAX = 24
_LIM = 1 << 62


def sat8(v):
    """Clamp to the symmetric int8 code range [-127, 127]."""
    return np.clip(np.asarray(v, dtype=np.int64), -127, 127)


def sat32(v):
    """Clamp to the int32 range."""
    return np.clip(np.asarray(v, dtype=np.int64), I32_MIN, I32_MAX)


def rshr(v, s):
    """Round-half-up arithmetic shift: floor(v * 2^-s + 1/2), elementwise.

    ``v`` is int64 with |v| < 2^62; ``s`` is an int or an int array.  For s < 0
    the exact product v * 2^-s is returned when it stays inside +-2^62 and is
    clamped to +-2^62 otherwise; every caller saturates to int32 afterwards, so
    the clamp never changes a result.
    """
    v = np.asarray(v, dtype=np.int64)
    s = np.asarray(s, dtype=np.int64)
    assert np.all(np.abs(v) < _LIM), "rshr operand out of range"
    if s.ndim == 0 and 1 <= int(s) <= 62:  # one shift for every element: no masks
        return (v + np.int64(1 << (int(s) - 1))) >> np.int64(s)
    v, s = np.broadcast_arrays(v, s)
    out = np.zeros(v.shape, dtype=np.int64)
    # s in [1, 62]: add half, arithmetic shift (numpy >> on int64 is floor division)
    m = (s >= 1) & (s <= 62)
    if np.any(m):
        sm = s[m]
        out[m] = (v[m] + np.left_shift(np.int64(1), sm - 1)) >> sm
    # s >= 63: |v| < 2^62 <= 2^(s-1), so the rounded quotient is 0 (already zero)
    m = s == 0
    out[m] = v[m]
    m = s < 0
    if np.any(m):
        k = -s[m]
        vm = v[m]
        big = k >= 62
        kk = np.where(big, 0, k)
        lim = np.right_shift(np.int64(_LIM), kk)
        r = np.left_shift(np.clip(vm, -lim, lim), kk)
        r = np.where(big, np.sign(vm) * _LIM, r)
        out[m] = r
    return out


def f32_to_i32_sat(f):
    """Integer-valued float32 array -> int64 values saturated to the int32 range."""
    f = np.asarray(f, dtype=np.float32).astype(np.float64)
    assert not np.any(np.isnan(f))
    return np.clip(f, I32_MIN, I32_MAX).astype(np.int64)


def pot_f32(a) -> int:
    """Exponent for a float32 tensor whose absolute maximum is ``a``.

    Largest p in [PMIN, PMAX] with a * 2^p <= 127; 0 when a == 0.
    """
    a = float(np.float32(a))
    assert a >= 0.0
    if a == 0.0:
        return 0
    for p in range(PMAX, PMIN - 1, -1):
        if a * (2.0 ** p) <= 127.0:
            return p
    return PMIN


def pot_q16(m) -> int:
    """Exponent for a Q.16 tensor (value = integer / 2^16) whose absolute maximum is ``m``.

    Largest p in [PMIN, PMAX] with (m / 2^16) * 2^p <= 127, i.e. the requantized
    codes rshr(v, 16 - p) stay inside [-127, 127]; 0 when m == 0.
    """
    m = int(m)
    assert m >= 0
    if m == 0:
        return 0
    for p in range(PMAX, PMIN - 1, -1):
        # m * 2^p <= 127 * 2^16, compared on exact integers
        if p >= 0:
            if m << p <= 127 << 16:
                return p
        else:
            if m <= (127 << 16) << (-p):
                return p
    return PMIN
