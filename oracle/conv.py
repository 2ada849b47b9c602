"""Power-of-two quantized causal depthwise conv1d with SiLU, and the x/B/C requant.

[FM] abstract and "What carries the argument": a fine-grained power-of-two
quantization serves the convolution layer and the SSM block; scales are 2^p,
so rescaling is a shift.  [FM] Fig. 2 (Mamba2 block flow): in_proj output
channels x|B|C pass a causal depthwise conv1d and SiLU before the SSM.

Readings:
* xBC (float32, the in_proj output columns of x, B and C) is quantized per
  tensor: p_c = pot(amax |xBC|) in dynamic mode (fixed in static mode),
  xBC_q = clamp(rint(xBC * 2^p_c), -127, 127), float32 product.
* Conv weights (offline): one exponent per channel, the "fine-grained" part:
  p_w[c] = pot(max_k |w[c, k]|), w_q = clamp(rint(w * 2^p_w[c]), -127, 127).
  The bias is kept in Q.16: b_q16 = sat32(rint(b * 2^16)).
* Causal padding: the d_conv-1 = 3 earlier inputs of each channel come from
  the conv cache (zeros for a fresh sequence).  acc = sum_k w_q[c,k] *
  xBC_q[t-3+k, c] in int32, then a = sat32(rshr(acc, p_c + p_w[c] - 16) + b_q16)
  in Q.16.
* SiLU in Q.16 (the NAU), then the channels split into x (d_inner), B and C
  (d_state each); each part gets its own exponent, p = pot_q16(amax) in
  dynamic mode, and codes rshr(s, 16 - p) clamped to [-127, 127].
"""
import numpy as np

from .fixedpoint import f32_to_i32_sat, pot_f32, pot_q16, rshr, sat8, sat32
from .nau import silu_q16


def conv_weight_prep(conv_w, conv_b):
    """Offline: per-channel power-of-two int8 conv weights and a Q.16 bias."""
    w = np.asarray(conv_w, dtype=np.float32)
    b = np.asarray(conv_b, dtype=np.float32)
    p_w = np.array([pot_f32(np.max(np.abs(w[c]))) for c in range(w.shape[0])], dtype=np.int64)
    scale = np.array([np.float32(2.0 ** int(p)) for p in p_w], dtype=np.float32)
    w_q = np.clip(np.rint(w * scale[:, None]), np.float32(-127), np.float32(127)).astype(np.int8)
    b_q16 = f32_to_i32_sat(np.rint(b * np.float32(65536.0)))
    return w_q, p_w, b_q16


def xbc_pot_quant(xbc, p_c=None):
    """Quantize the conv input; ``p_c`` None means dynamic (from the tensor's max).

    Returns (xbc_q int8, p_c, amax float32).
    """
    xbc = np.asarray(xbc, dtype=np.float32)
    amax = np.float32(np.max(np.abs(xbc))) if xbc.size else np.float32(0.0)
    if p_c is None:
        p_c = pot_f32(amax)
    q = np.clip(np.rint(xbc * np.float32(2.0 ** int(p_c))), np.float32(-127),
                np.float32(127)).astype(np.int8)
    return q, int(p_c), amax


def conv1d_pot(xbc_q, w_q, p_w, b_q16, p_c, state_in=None):
    """Causal depthwise conv over time on int8 codes, output in Q.16.

    xbc_q [B, L, ch] int8; w_q [ch, 4]; p_w [ch]; b_q16 [ch];
    state_in [B, ch, 3] int8 (inputs at t = -3, -2, -1, oldest first) or None.
    Returns (a int64 [B, L, ch] Q.16, acc int64 [B, L, ch], state_out [B, ch, 3] int8).
    """
    xq = np.asarray(xbc_q, dtype=np.int64)
    Bsz, L, ch = xq.shape
    K = w_q.shape[1]
    assert K == 4
    if state_in is None:
        prev = np.zeros((Bsz, K - 1, ch), dtype=np.int64)
    else:
        prev = np.transpose(np.asarray(state_in, dtype=np.int64), (0, 2, 1))
    padded = np.concatenate([prev, xq], axis=1)          # [B, L+3, ch]
    w = np.asarray(w_q, dtype=np.int64)
    acc = np.zeros((Bsz, L, ch), dtype=np.int64)
    for k in range(K):
        acc += w[None, None, :, k] * padded[:, k:k + L, :]
    shift = int(p_c) + np.asarray(p_w, dtype=np.int64) - 16
    a = sat32(rshr(acc, shift[None, None, :]) + np.asarray(b_q16, dtype=np.int64)[None, None, :])
    state_out = np.transpose(padded[:, L:L + K - 1, :], (0, 2, 1)).astype(np.int8)
    return a, acc, state_out


def silu_requant(a, d_inner, dstate, p_fixed=None):
    """SiLU in Q.16, split into x / B / C, per-part power-of-two int8 codes.

    ``p_fixed`` None: dynamic exponents from each part's max; otherwise a
    (p_x, p_B, p_C) triple (static mode, or exponents frozen for decode).
    Returns (x_q, B_q, C_q int8, (p_x, p_B, p_C), (amax_x, amax_B, amax_C) Q.16, s).
    """
    s = silu_q16(a)
    parts = (s[..., :d_inner], s[..., d_inner:d_inner + dstate], s[..., d_inner + dstate:])
    assert parts[2].shape[-1] == dstate
    amaxes = tuple(int(np.max(np.abs(p))) if p.size else 0 for p in parts)
    if p_fixed is None:
        ps = tuple(pot_q16(m) for m in amaxes)
    else:
        ps = tuple(int(p) for p in p_fixed)
    codes = tuple(sat8(rshr(part, 16 - p)).astype(np.int8) for part, p in zip(parts, ps))
    return codes[0], codes[1], codes[2], ps, amaxes, s
