"""Quantization statistics of the layer's activation quantization points.

TEST INFRASTRUCTURE (see the package docstring).

[FM] referee report, major comment on Sections III-A / IV-B, and [FMV] skeptic
critique: Algorithm 1 takes each scale from the current input's maximum, the
hardware of Fig. 6 multiplies by a fixed calibrated (scoe, sshift); how often
the fixed scale clips, and how much error either adds, is the open question.
These functions measure both at one point: for every element, its value v, its
int8 code q (clamped to [-127, 127]) and the code's step (the dequant scale),
whether the rounded code left the range before the clamp, and the
dequantization error v - q * step, accumulated in float64.

Points (the order of fm_quant_stats): u and g are the two Hadamard points
(in_proj and out_proj inputs, after the rotation); xBC is the conv input;
x, B, C are the SiLU outputs feeding the scan (values Q.16 / 2^16).
"""
import numpy as np

from .fixedpoint import rshr, sat8

POINTS = ("u", "g", "xbc", "x", "B", "C")


def _summary(v, q, step, clipped):
    v = np.asarray(v, dtype=np.float64).ravel()
    e = v - np.asarray(q, dtype=np.float64).ravel() * np.float64(step)
    return {"count": int(v.size), "clipped": int(np.count_nonzero(clipped)),
            "sq_err": float(np.sum(e * e)), "sq_val": float(np.sum(v * v))}


def hadamard_point_stats(r, c):
    """Rotated values r under the float32 multiplier c: q = sat8(rint(r * c)), step 1/c."""
    c = np.float32(c)
    rc = np.rint(np.asarray(r, np.float32) * c)          # float32 product, then rint
    q = np.clip(rc, np.float32(-127), np.float32(127))
    step = np.float32(np.float32(1.0) / c)                # the dequant scale as stored
    return _summary(r, q, step, np.abs(rc) > 127)


def pot_float_point_stats(v, p):
    """Float values v with the power-of-two scale 2^p: q = sat8(rint(v * 2^p)), step 2^-p."""
    vp = np.rint(np.asarray(v, np.float32) * np.float32(2.0 ** int(p)))
    q = np.clip(vp, np.float32(-127), np.float32(127))
    return _summary(v, q, 2.0 ** -int(p), np.abs(vp) > 127)


def pot_q16_point_stats(s, p):
    """Q.16 integers s (value s / 2^16) with exponent p: q = sat8(rshr(s, 16 - p)), step 2^-p."""
    s = np.asarray(s, dtype=np.int64)
    qr = rshr(s, 16 - int(p))
    return _summary(s.astype(np.float64) * 2.0 ** -16, sat8(qr), 2.0 ** -int(p), np.abs(qr) > 127)


def empty():
    return {k: {"count": 0, "clipped": 0, "sq_err": 0.0, "sq_val": 0.0} for k in POINTS}


def accumulate(into, point, st):
    """Add one point's statistics into a POINTS-keyed dict (as the device record adds)."""
    d = into[point]
    for k in ("count", "clipped", "sq_err", "sq_val"):
        d[k] += st[k]
    return into
