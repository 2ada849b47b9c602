"""The outlier study's three W8A8 schemes for one linear layer y = x w^T.

TEST INFRASTRUCTURE (see the package docstring).

[FM] abstract, Fig. 3 caption and Table II: the Hadamard rotation is what lets
8-bit linear layers keep activations with outliers; [MPTQ] abstract: the
outliers sit in a few channels.  The comparison takes the same layer three
ways, every scheme dynamic and per tensor:
* "hadamard" (the method): x H and w H quantized (hadamard.hadamard_quant,
  linear.quantize_weight), int8 GEMM, dequantized;
* "naive": x and w quantized as they are;
* "smooth" (SmoothQuant-style, alpha = 1/2): per input channel j,
  s_j = sqrt(max_i |x_ij|) / sqrt(max_r |w_rj|) (1 if either is 0);
  x / s and w * s quantized.
Reading: both maxima, the square roots and the quotient are float32 with
IEEE rounding (correctly rounded sqrt and division), as the kernels compute.
"""
import numpy as np

from .hadamard import hadamard_quant
from .linear import quantize_weight, w8a8_gemm


def per_tensor_quant(x):
    """q = sat8(rint(x * c)), c = 127 / max|x| (1 if 0), scale 1/c, all float32."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    c = np.float32(1.0) if amax == 0 else np.float32(127.0) / amax
    q = np.clip(np.rint(x * c), np.float32(-127), np.float32(127)).astype(np.int8)
    return q, np.float32(np.float32(1.0) / c)


def smooth_scales(x, w):
    """s_j = sqrt(max_i |x_ij|) / sqrt(max_r |w_rj|), float32 (1 where a max is 0)."""
    ax = np.max(np.abs(np.asarray(x, np.float32)), axis=0)
    aw = np.max(np.abs(np.asarray(w, np.float32)), axis=0)
    ok = (ax > 0) & (aw > 0)
    s = np.ones(ax.shape, np.float32)
    s[ok] = (np.sqrt(ax[ok]) / np.sqrt(aw[ok])).astype(np.float32)
    return s


def scheme(x, w, name):
    """Codes, scales and the dequantized output of one scheme.

    Returns dict(a, s_a (activation codes and scale, in the scheme's domain),
    b, s_b (weight codes and scale), xs (the activations the codes quantize),
    out float32 [rows, n]).
    """
    x = np.asarray(x, np.float32)
    w = np.asarray(w, np.float32)
    if name == "hadamard":
        a, s_a, _, xs = hadamard_quant(x, "dynamic")
        b, s_b = quantize_weight(w)
    elif name == "naive":
        xs = x
        a, s_a = per_tensor_quant(x)
        b, s_b = per_tensor_quant(w)
    elif name == "smooth":
        s = smooth_scales(x, w)
        xs = (x / s).astype(np.float32)
        a, s_a = per_tensor_quant(xs)
        b, s_b = per_tensor_quant((w * s).astype(np.float32))
    else:
        raise ValueError(name)
    _, out = w8a8_gemm(a, b, s_a, s_b)
    return {"a": a, "s_a": s_a, "b": b, "s_b": s_b, "xs": xs, "out": out}


def output_error(out, x, w):
    """||out - x w^T|| / ||x w^T|| with the reference product in float64."""
    ref = np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
    return float(np.linalg.norm(np.asarray(out, np.float64) - ref) / np.linalg.norm(ref))


def activation_sqnr_db(codes, scale, xs):
    """10 log10(sum xs^2 / sum (xs - codes * scale)^2) in the scheme's domain."""
    xs = np.asarray(xs, np.float64)
    e = xs - np.asarray(codes, np.float64) * np.float64(scale)
    return float(10 * np.log10(np.sum(xs * xs) / np.sum(e * e)))
