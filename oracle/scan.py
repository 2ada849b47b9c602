"""dt / decay through the NAU, and the fixed-point selective scan.

[FM] "What carries the argument": power-of-two scaling makes the SSM block's
arithmetic shifts, adds and products; [FMV] supporting citations [14]
(zero-order-hold discretization, giving the decay e^(dt*A)) and [15] (the
shift-based exponential used for e^dt).  [FM] Fig. 2: per head, the state
h[p, n] evolves as h_t = exp(dt_t * A) h_{t-1} + dt_t * x_t[p] * B_t[n] and the
output is y_t[p] = sum_n C_t[n] h_t[p, n] + D x_t[p] (Mamba2, one group).

Readings:
* dt_in = sat32(rint((dt_raw + dt_bias) * 2^16)) (float32 add, then the exact
  scaling); dt = SoftPlus(dt_in) in Q.16; A_q16 = sat32(rint(A * 2^16));
  dA = e^(rshr(dt * A_q16, 16)) in Q.16 (argument <= 0, so dA in [0, 2^16]).
* Exponents: x has p_x, B has p_B, C has p_C.  The state is int32 with
  exponent p_h = p_x + p_B + 8 and the output y is int32 with exponent
  p_y = p_x + 8.
* One step, per (batch, head, p, n), in exact integers:
    u   = dt * x_q                                   (exponent 16 + p_x)
    h_t = sat32( floor( (dA * h_{t-1} + 2^8 * u * B_q + 2^15) / 2^16 ) )
  i.e. the decayed state and the input term are aligned to exponent
  16 + p_h, summed exactly and rounded half up once onto the state grid.
    y_acc = sum_n C_q * h_t                          (exponent p_C + p_h)
    y     = sat32( rshr(y_acc, p_B + p_C) + rshr(D_q16 * x_q, 8) )
* The scan is sequential in t; the state starts at zero or from the cache.
"""
import numpy as np

from .fixedpoint import f32_to_i32_sat, rshr, sat32
from .nau import exp_q16, softplus_q16


def dt_dA(dt_raw, dt_bias, A_q16):
    """dt_raw [..., H] float32 -> (dt Q.16, dA Q.16) int64 arrays of the same shape."""
    dt_raw = np.asarray(dt_raw, dtype=np.float32)
    dt_in = f32_to_i32_sat(np.rint((dt_raw + np.asarray(dt_bias, dtype=np.float32))
                                   * np.float32(65536.0)))
    dt = softplus_q16(dt_in)
    arg = sat32(rshr(dt * np.asarray(A_q16, dtype=np.int64), 16))
    assert np.all(arg <= 0), "A must be <= 0"
    dA = exp_q16(arg)
    return dt, dA


def ssm_scan_pot(x_q, B_q, C_q, dt, dA, D_q16, p_B, p_C, state_in=None):
    """Fixed-point scan.

    x_q [Bsz, L, H, P] int8; B_q, C_q [Bsz, L, N] int8; dt, dA [Bsz, L, H] Q.16;
    D_q16 [H]; state_in [Bsz, H, P, N] int32 or None.
    Returns (y int64 [Bsz, L, H, P], state_out int64 [Bsz, H, P, N]).
    """
    x = np.asarray(x_q, dtype=np.int64)
    Bm = np.asarray(B_q, dtype=np.int64)
    Cm = np.asarray(C_q, dtype=np.int64)
    dt = np.asarray(dt, dtype=np.int64)
    dA = np.asarray(dA, dtype=np.int64)
    D = np.asarray(D_q16, dtype=np.int64)
    Bsz, L, H, P = x.shape
    N = Bm.shape[-1]
    if state_in is None:
        h = np.zeros((Bsz, H, P, N), dtype=np.int64)
    else:
        h = np.asarray(state_in, dtype=np.int64).copy()
    y = np.zeros((Bsz, L, H, P), dtype=np.int64)
    ky = int(p_B) + int(p_C)
    for t in range(L):
        u = dt[:, t, :, None] * x[:, t]                                  # [Bsz, H, P]
        inc = (u[..., None] * Bm[:, t, None, None, :]) << 8              # [Bsz, H, P, N]
        num = dA[:, t, :, None, None] * h + inc + (1 << 15)
        h = sat32(num >> 16)
        y_acc = np.sum(Cm[:, t, None, None, :] * h, axis=-1)            # exact int64
        y[:, t] = sat32(rshr(y_acc, ky) + rshr(D[None, :, None] * x[:, t], 8))
    return y, h


# --- narrower state cache ----------------------------------------------------
# The state width sets the decode step's memory traffic (the state is read and
# written once per token).  Reading for a cache narrower than int32, in the
# method's own power-of-two idiom: the cache holds codes c of `bits` bits on
# the coarser grid 2^shift of the state's own (exponent p_h - shift), rounded
# half up and saturated:
#     c = clamp(floor((h + 2^(shift-1)) / 2^shift), -2^(bits-1), 2^(bits-1) - 1)
# (no rounding term when shift = 0); a step widens the cache to h = c * 2^shift,
# takes the exact step of ssm_scan_pot (its y from the int32 state of the step)
# and narrows the new state for the cache.  Stored layout: int16, or the low 24
# bits of the two's-complement code as three little-endian bytes, in the state's
# [batch, nheads, headdim, dstate] order.

STATE_BITS = (16, 24)


def narrow_state(h, bits, shift):
    """int32 state values -> cache codes of `bits` bits on the grid 2^shift."""
    assert bits in STATE_BITS and 0 <= shift <= 32 - bits
    h = np.asarray(h, dtype=np.int64)
    c = (h + ((1 << shift) >> 1)) >> shift        # floor division: half up
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    return np.clip(c, lo, hi)


def widen_state(c, shift):
    """Cache codes -> state values on the int32 grid (exact: c * 2^shift)."""
    return np.asarray(c, dtype=np.int64) << shift


def pack_state(c, bits):
    """Codes -> the stored bytes (little endian, 2 or 3 bytes per value)."""
    c = np.asarray(c, dtype=np.int64).reshape(-1)
    nb = bits // 8
    u = c & ((1 << bits) - 1)
    out = np.zeros((c.size, nb), dtype=np.uint8)
    for k in range(nb):
        out[:, k] = (u >> (8 * k)) & 0xFF
    return out.reshape(-1)


def unpack_state(buf, bits):
    """The stored bytes -> codes (sign-extended from `bits`)."""
    nb = bits // 8
    b = np.asarray(buf, dtype=np.uint8).reshape(-1, nb).astype(np.int64)
    u = np.zeros(b.shape[0], dtype=np.int64)
    for k in range(nb):
        u |= b[:, k] << (8 * k)
    return np.where(u >= (1 << (bits - 1)), u - (1 << bits), u)


def state_shift_for(amax, bits, headroom=1):
    """Smallest shift whose codes hold |h| <= amax * 2^headroom without clipping:
    max(0, bitlength(amax) + headroom - (bits - 1)), at most 32 - bits."""
    need = int(amax).bit_length() + int(headroom)
    return min(max(0, need - (bits - 1)), 32 - bits)


# --- the chunked (SSD-form) variant: the real recurrence -----------------------
# A chunked scan sums the recurrence in matrix form over chunks of tokens, so it
# cannot reproduce the per-step rounding above; what it computes exactly (up to
# the order of its float64 roundings) is the recurrence with that rounding left
# out.  Reading: in the state's own grid units, with a_t = dA_t / 2^16,
#     h_t = a_t * h_{t-1} + dt_t * x_t[p] * B_t[n] / 2^8      (no rounding)
#     y_t = sat32(floor(sum_n C_t[n] h_t / 2^(p_B + p_C) + 1/2) + rshr(D x_t, 8))
# and the final state is h rounded half up onto the grid and saturated.  No
# saturation happens inside the sequence (inputs whose exact state saturates lie
# outside the variant's contract).


def ssm_scan_real(x_q, B_q, C_q, dt, dA, D_q16, p_B, p_C, state_in=None):
    """The recurrence without per-step rounding, in float64, t ascending.

    Same arguments as ssm_scan_pot.  Returns (y int64, state_out int64, y_acc
    float64 [Bsz, L, H, P] = sum_n C h before the output rounding)."""
    x = np.asarray(x_q, dtype=np.float64)
    Bm = np.asarray(B_q, dtype=np.float64)
    Cm = np.asarray(C_q, dtype=np.float64)
    a = np.asarray(dA, dtype=np.float64) / 65536.0
    dtf = np.asarray(dt, dtype=np.float64)
    Bsz, L, H, P = x.shape
    N = Bm.shape[-1]
    h = (np.zeros((Bsz, H, P, N)) if state_in is None
         else np.asarray(state_in, dtype=np.float64).copy())
    y_acc = np.zeros((Bsz, L, H, P))
    for t in range(L):
        u = dtf[:, t, :, None] * x[:, t] / 256.0                          # [Bsz, H, P]
        h = a[:, t, :, None, None] * h + u[..., None] * Bm[:, t, None, None, :]
        y_acc[:, t] = np.einsum("bn,bhpn->bhp", Cm[:, t], h)
    ky = int(p_B) + int(p_C)
    xi = np.asarray(x_q, dtype=np.int64)
    yd = rshr(np.asarray(D_q16, dtype=np.int64)[None, None, :, None] * xi, 8)
    big = 2.0 ** 62  # beyond the int32 range either way: clip before converting
    y = sat32(np.clip(np.floor(y_acc * 2.0 ** -ky + 0.5), -big, big).astype(np.int64) + yd)
    st = sat32(np.clip(np.floor(h + 0.5), -big, big).astype(np.int64))
    return y, st, y_acc
