"""Output gate, gated RMSNorm and the out_proj input quantization.

[FM] Fig. 2 (Mamba2 block flow): the SSM output is gated by SiLU(z), passed
through RMSNorm (the pages cite RMSNorm as their ref. [10] and SiLU as [11])
and projected by out_proj, whose input is Hadamard-rotated and quantized to
int8 like the in_proj input ("What carries the argument").

Readings:
* Gate (the Mamba2 gated norm with the norm after the gate, one group):
  y_f = float32(y) * 2^-p_y; z_q = sat32(rint(z * 2^16)); the gate value is
  float32(SiLU_q16(z_q)) * 2^-16 from the NAU; g = y_f * gate (float32).
* RMSNorm over d_inner in float32, in one fixed summation order, because the
  normed values are turned into int8 codes and any rounding change can flip a
  code: 64 partial sums, partial l adding g_i * g_i for i = l, l+64, l+128, ...
  in ascending order (each square rounded, then added: no fused multiply-add);
  then partial sums combined pairwise across index distance 32, 16, 8, 4, 2, 1
  (a[l] += a[l xor k]); ss = a[0].  ms = ss / D, r = 1 / sqrt(ms + 1e-5),
  n_i = (g_i * r) * w_i.  Division and square root correctly rounded.
"""
import numpy as np

from .fixedpoint import f32_to_i32_sat
from .hadamard import hadamard_quant
from .nau import silu_q16

EPS = np.float32(1e-5)


def gate(y, z, p_y):
    """y int [T, D] with exponent p_y, z float32 [T, D] -> g float32 [T, D]."""
    y_f = np.asarray(y, dtype=np.int64).astype(np.float32) * np.float32(2.0 ** (-int(p_y)))
    z_q = f32_to_i32_sat(np.rint(np.asarray(z, dtype=np.float32) * np.float32(65536.0)))
    sz = silu_q16(z_q).astype(np.float32) * np.float32(2.0 ** -16)
    return y_f * sz


def rmsnorm_fixed_order(g, w, eps=EPS):
    """Row-wise RMSNorm of float32 [T, D] (D % 64 == 0) in the fixed order above."""
    g = np.asarray(g, dtype=np.float32)
    T, D = g.shape
    assert D % 64 == 0
    sq = g * g
    a = np.zeros((T, 64), dtype=np.float32)
    for j in range(D // 64):
        a = a + sq[:, j * 64:(j + 1) * 64]
    lanes = np.arange(64)
    for k in (32, 16, 8, 4, 2, 1):
        a = a + a[:, lanes ^ k]
    ss = a[:, 0]
    ms = ss / np.float32(D)
    r = np.float32(1.0) / np.sqrt(ms + np.float32(eps))
    return (g * r[:, None]) * np.asarray(w, dtype=np.float32)[None, :]


def gate_norm_quant(y, z, p_y, norm_w, mode="dynamic", scoe=None, sshift=None):
    """Gate, RMSNorm, then Hadamard rotation + per-tensor int8 of the result.

    Returns (g_q int8, s_g float32, amax float32, normed float32).
    """
    n = rmsnorm_fixed_order(gate(y, z, p_y), norm_w)
    q, s, amax, _ = hadamard_quant(n, mode, scoe, sshift)
    return q, s, amax, n
