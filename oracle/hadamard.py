"""Hadamard rotation and per-tensor int8 quantization.

[FM] "What carries the argument": the linear layer is factored as
Y = (X H)(H^T W^T) with H a Hadamard matrix normalized by sqrt(n), which is
orthonormal, so rotating activations and weights leaves Y unchanged while
spreading outlier energy.  [FM] referee report, major comment on Sections
III-A / IV-B: Algorithm 1 takes the activation and weight scales from the
maximum of the rotated tensors (an input-dependent, two-pass step), while the
Hadamard linear module of Fig. 6 applies a fixed multiply ("x scoe") and
shift (">> sshift") with no max unit.  [FMV] skeptic critique: static scales
calibrated offline and applied by multiply+shift.

Readings (the pages leave these open):
* H_K for a row of length K (K a multiple of 256) is block-diagonal, K/256
  copies of S_256 / 16, S_256 the Sylvester Hadamard matrix in natural order
  (symmetric, so H^T = H).  FindHadamard of Algorithm 1 depends only on the
  dimension.
* The transform runs as a radix-2 fast Walsh-Hadamard transform in float32,
  stages h = 1, 2, 4, ..., 128 in that order, butterfly (a, b) -> (a+b, a-b),
  then the exact scaling by 1/16.
* Scale granularity is per tensor (the whole call), symmetric:
  dynamic  c = 127 / amax   (one IEEE float32 division; amax = 0 gives c = 1)
  static   c = scoe * 2^-sshift
  codes q = clamp(rint(r * c), -127, 127) with rint half-to-even, float32
  product; the dequantization scale is s = 1 / c (float32).
"""
import numpy as np


def fwht256_f32(x):
    """Rows of ``x`` (float32 [..., K], K % 256 == 0) times H_K, in float32."""
    x = np.asarray(x, dtype=np.float32)
    K = x.shape[-1]
    assert K % 256 == 0, "row length must be a multiple of the 256-wide Hadamard block"
    v = x.reshape(-1, 256).copy()
    h = 1
    while h < 256:
        # element j of a block = g*2h + bit*h + i : pair (j, j+h) for j with bit h clear
        v = v.reshape(-1, 256 // (2 * h), 2, h)
        a = v[:, :, 0, :]
        b = v[:, :, 1, :]
        v = np.stack((a + b, a - b), axis=2)
        h *= 2
    return v.reshape(x.shape) * np.float32(0.0625)


def hadamard_scale(amax, mode="dynamic", scoe=None, sshift=None):
    """The float32 multiplier c of the quantizer (dynamic: from the tensor max)."""
    amax = np.float32(amax)
    if mode == "dynamic":
        c = np.float32(1.0) if amax == 0 else np.float32(127.0) / amax
    elif mode == "static":
        assert scoe is not None and sshift is not None and 0 < scoe < (1 << 24)
        assert -126 <= sshift <= 126
        c = np.float32(scoe) * np.float32(2.0 ** (-sshift))
    else:
        raise ValueError(mode)
    return np.float32(c)


def quantize_codes(r, c):
    """int8 codes of the rotated values ``r`` under multiplier ``c``, and s = 1/c."""
    c = np.float32(c)
    # clamp while still float (static scales can send r*c far outside int range)
    q = np.clip(np.rint(np.asarray(r, np.float32) * c), np.float32(-127),
                np.float32(127)).astype(np.int8)
    return q, np.float32(np.float32(1.0) / c)


def hadamard_quant(x, mode="dynamic", scoe=None, sshift=None):
    """Rotate the rows of ``x`` by H_K and quantize the whole tensor to int8.

    Returns (q int8, s float32 dequant scale, amax float32 of the rotated
    tensor, r float32 rotated tensor).
    """
    r = fwht256_f32(x)
    amax = np.float32(np.max(np.abs(r))) if r.size else np.float32(0.0)
    q, s = quantize_codes(r, hadamard_scale(amax, mode, scoe, sshift))
    return q, s, amax, r
