"""W8A8 linear layers (in_proj, out_proj).

[FM] abstract and referee summary: the linear layers run with 8-bit weights
and activations after the Hadamard rotation; [FM] "What carries the argument":
Y = (X H)(H^T W^T).

Readings: the weight rotation applies H along the input dimension of every
weight row (W H, i.e. H^T W^T as a right factor), then the same per-tensor
dynamic quantization as the activations.  The product accumulates in int32
(exact: |acc| <= K * 127^2 < 2^31 for K <= 133144) and is dequantized as
float(acc) * (s_a * s_b), the two scales multiplied first in float32.
"""
import numpy as np

from .hadamard import hadamard_quant


def quantize_weight(w):
    """Offline weight preparation: rotate rows along K, per-tensor int8."""
    q, s, _, _ = hadamard_quant(np.asarray(w, dtype=np.float32), mode="dynamic")
    return q, s


def w8a8_gemm(a_q, b_q, s_a, s_b):
    """acc = a_q @ b_q^T in exact integers; out = float32(acc) * (s_a * s_b).

    a_q [M, K] int8, b_q [N, K] int8.  Returns (acc int64 [M, N], out float32).
    The float64 matrix product is exact here: every partial sum is an integer
    below 2^53.
    """
    a = np.asarray(a_q, dtype=np.int8)
    b = np.asarray(b_q, dtype=np.int8)
    assert a.shape[1] == b.shape[1]
    assert a.shape[1] * 127 * 127 < (1 << 31)
    acc = (a.astype(np.float64) @ b.astype(np.float64).T).astype(np.int64)
    s_ab = np.float32(s_a) * np.float32(s_b)
    out = acc.astype(np.float32) * s_ab
    return acc, out
