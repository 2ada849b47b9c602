"""The quantized Mamba2 mixer layer end to end: prefill, decode, stacks, calibration.

[FM] Fig. 2 (Mamba2 block flow): in_proj -> causal conv1d -> SiLU -> SSM ->
gated RMSNorm -> out_proj.  [FM] referee summary: W8A8 linear layers with the
Hadamard rotation, power-of-two quantization in the conv and SSM, linear
approximations of exp and SoftPlus.  [FM] major comment on Sections III-A /
IV-B and [FMV] skeptic critique: dynamic (max-based, per input) scales as in
Algorithm 1, or static scales calibrated on a set of inputs and applied by
multiply+shift as in the hardware of Fig. 6.

Readings:
* in_proj output columns are split [z | x | B | C | dt] (Mamba2 order).
* Static mode fixes every activation quantization point of the layer: the two
  Hadamard points (in_proj input, out_proj input) by (scoe, sshift), and the
  four power-of-two points (xBC, x, B, C) by their exponents.  Calibration
  runs the dynamic path over the calibration inputs, keeps the maximum seen at
  each point, and converts: c = 127 / amax (float64), sshift chosen so that
  2^14 <= c * 2^sshift < 2^15, scoe = rint(c * 2^sshift); p = pot(amax).
* Stacks are pre-norm residual: h <- h + mixer(RMSNorm(h)), the RMSNorm over
  d_model with weight 1 and the fixed summation order of gate_norm.
* Decode takes one token per sequence: the conv window and the int32 state
  come from the cache, the four power-of-two exponents are frozen in the
  cache by the prefill that filled it, and the Hadamard scales follow the
  layer mode (dynamic: per tensor over the batch rows of the step).
"""
from dataclasses import dataclass, field

import numpy as np

from .conv import conv1d_pot, conv_weight_prep, silu_requant, xbc_pot_quant
from .fixedpoint import f32_to_i32_sat, pot_f32, pot_q16
from .gate_norm import gate, rmsnorm_fixed_order
from . import quant_stats as QS
from .hadamard import hadamard_quant, hadamard_scale
from .linear import quantize_weight, w8a8_gemm
from .scan import dt_dA, narrow_state, ssm_scan_pot, widen_state


@dataclass
class QParams:
    """Static quantization parameters of one layer."""
    scoe: tuple = (1 << 14, 1 << 14)     # (in_proj input, out_proj input)
    sshift: tuple = (14, 14)
    p: tuple = (0, 0, 0, 0)              # (p_c, p_x, p_B, p_C)


@dataclass
class Stats:
    """Maxima observed at the quantization points (calibration)."""
    amax_u: float = 0.0
    amax_g: float = 0.0
    amax_xbc: float = 0.0
    amax_q16: list = field(default_factory=lambda: [0, 0, 0])   # x, B, C (Q.16 integers)

    def update(self, other: "Stats") -> None:
        self.amax_u = max(self.amax_u, other.amax_u)
        self.amax_g = max(self.amax_g, other.amax_g)
        self.amax_xbc = max(self.amax_xbc, other.amax_xbc)
        self.amax_q16 = [max(a, b) for a, b in zip(self.amax_q16, other.amax_q16)]


def prepare_layer(params: dict) -> dict:
    """Offline parameter preparation (not part of the timed path)."""
    w_in_q, s_w_in = quantize_weight(params["w_in"])
    w_out_q, s_w_out = quantize_weight(params["w_out"])
    conv_w_q, p_w, b_q16 = conv_weight_prep(params["conv_w"], params["conv_b"])
    return {
        "w_in_q": w_in_q, "s_w_in": s_w_in,
        "w_out_q": w_out_q, "s_w_out": s_w_out,
        "conv_w_q": conv_w_q, "p_w": p_w, "conv_b_q16": b_q16,
        "dt_bias": np.asarray(params["dt_bias"], dtype=np.float32),
        "A_q16": f32_to_i32_sat(np.rint(np.asarray(params["A"], np.float32) * np.float32(65536))),
        "D_q16": f32_to_i32_sat(np.rint(np.asarray(params["D"], np.float32) * np.float32(65536))),
        "norm_w": np.asarray(params["norm_w"], dtype=np.float32),
    }


def _mixer(prep, shape, u2, Bsz, L, mode, qp, cache_in, frozen_p, collect=False, scan=None):
    """Shared body of prefill (L tokens) and decode (L = 1) on rows u2 [Bsz*L, dm].

    ``collect``: also return the quantization statistics of the six points in
    r["qstats"] (oracle.quant_stats).
    """
    s = shape
    di, N, H, P, ch = s.d_inner, s.dstate, s.nheads, s.headdim, s.conv_ch
    r = {}
    st = Stats()
    hq_mode = "static" if mode == "static" else "dynamic"
    sc0 = (qp.scoe[0], qp.sshift[0]) if hq_mode == "static" else (None, None)
    u_q, s_u, amax_u, u_rot = hadamard_quant(u2, hq_mode, *sc0)
    acc_in, v = w8a8_gemm(u_q, prep["w_in_q"], s_u, prep["s_w_in"])
    r.update(u_q=u_q, s_u=s_u, acc_in=acc_in, v=v)
    st.amax_u = float(amax_u)
    z = v[:, :di]
    xbc = v[:, di:di + ch]
    dt_raw = v[:, di + ch:di + ch + H]
    if frozen_p is not None:
        p_fixed = tuple(int(p) for p in frozen_p)
    elif mode == "static":
        p_fixed = tuple(int(p) for p in qp.p)
    else:
        p_fixed = None
    xbc_q, p_c, amax_xbc = xbc_pot_quant(xbc, None if p_fixed is None else p_fixed[0])
    st.amax_xbc = float(amax_xbc)
    conv_state_in = None if cache_in is None else cache_in["conv_state"]
    a, conv_acc, conv_state = conv1d_pot(xbc_q.reshape(Bsz, L, ch), prep["conv_w_q"], prep["p_w"],
                                         prep["conv_b_q16"], p_c, conv_state_in)
    x_q, B_q, C_q, (p_x, p_B, p_C), amaxes, silu_a = silu_requant(
        a, di, N, None if p_fixed is None else p_fixed[1:])
    st.amax_q16 = list(amaxes)
    dt, dA = dt_dA(dt_raw.reshape(Bsz, L, H), prep["dt_bias"], prep["A_q16"])
    state_in = None if cache_in is None else cache_in["ssm_state"]
    y, state = (scan or ssm_scan_pot)(x_q.reshape(Bsz, L, H, P), B_q, C_q, dt, dA,
                                      prep["D_q16"], p_B, p_C, state_in)
    p_y = p_x + 8
    sc1 = (qp.scoe[1], qp.sshift[1]) if hq_mode == "static" else (None, None)
    g = gate(y.reshape(Bsz * L, di), z, p_y)
    normed = rmsnorm_fixed_order(g, prep["norm_w"])
    g_q, s_g, amax_g, g_rot = hadamard_quant(normed, hq_mode, *sc1)
    st.amax_g = float(amax_g)
    acc_out, out = w8a8_gemm(g_q, prep["w_out_q"], s_g, prep["s_w_out"])
    r.update(z=z, xbc=xbc, dt_raw=dt_raw, xbc_q=xbc_q, conv_acc=conv_acc, conv_a=a,
             silu=silu_a, x_q=x_q, B_q=B_q, C_q=C_q, p=(p_c, p_x, p_B, p_C), dt=dt, dA=dA,
             y=y, g=g, normed=normed, g_q=g_q, s_g=s_g, acc_out=acc_out)
    if collect:
        qs = QS.empty()
        QS.accumulate(qs, "u", QS.hadamard_point_stats(u_rot, hadamard_scale(amax_u, hq_mode, *sc0)))
        QS.accumulate(qs, "g", QS.hadamard_point_stats(g_rot, hadamard_scale(amax_g, hq_mode, *sc1)))
        QS.accumulate(qs, "xbc", QS.pot_float_point_stats(xbc, p_c))
        s_all = silu_a.reshape(-1, ch)
        QS.accumulate(qs, "x", QS.pot_q16_point_stats(s_all[:, :di], p_x))
        QS.accumulate(qs, "B", QS.pot_q16_point_stats(s_all[:, di:di + N], p_B))
        QS.accumulate(qs, "C", QS.pot_q16_point_stats(s_all[:, di + N:], p_C))
        r["qstats"] = qs
    cache = {"conv_state": conv_state, "ssm_state": state,
             "p": np.array([p_c, p_x, p_B, p_C], dtype=np.int64)}
    return out, r, cache, st


def layer_prefill(prep, shape, u, mode="dynamic", qp=None, collect=False, scan=None):
    """One mixer layer over u [Bsz, L, d_model] from a fresh state.

    Returns (out float32 [Bsz, L, d_model], intermediates, cache, stats);
    ``collect`` adds the quantization statistics as intermediates["qstats"];
    ``scan``: another implementation of scan.ssm_scan_pot (scan_c's, for full
    sizes).
    """
    u = np.asarray(u, dtype=np.float32)
    Bsz, L, dm = u.shape
    out, r, cache, st = _mixer(prep, shape, u.reshape(Bsz * L, dm), Bsz, L, mode, qp, None, None,
                               collect, scan)
    return out.reshape(Bsz, L, dm), r, cache, st


def layer_decode(prep, shape, u_t, cache, mode="dynamic", qp=None, state_fmt=None):
    """One token per sequence, u_t [Bsz, d_model], continuing from ``cache``.

    ``state_fmt`` = (bits, shift): the cache's "ssm_state" holds narrow codes
    (scan.narrow_state); the step widens them, runs as with an int32 state, and
    narrows the new state into the returned cache."""
    u_t = np.asarray(u_t, dtype=np.float32)
    Bsz, dm = u_t.shape
    if state_fmt is not None:
        bits, shift = state_fmt
        cache = dict(cache, ssm_state=widen_state(cache["ssm_state"], shift))
    out, r, new_cache, st = _mixer(prep, shape, u_t, Bsz, 1, mode, qp, cache, cache["p"])
    if state_fmt is not None:
        new_cache["ssm_state"] = narrow_state(new_cache["ssm_state"], bits, shift)
    return out.reshape(Bsz, dm), r, new_cache, st


def stack_prefill(preps, shape, u, mode="dynamic", qps=None, qstats=None, scan=None):
    """Pre-norm residual stack over u [Bsz, L, d_model].

    Returns (h float32 [Bsz, L, d_model], caches, stats per layer).  ``qstats``
    (a list, one oracle.quant_stats dict per layer) receives each layer's
    quantization statistics added in; ``scan`` as in layer_prefill.
    """
    h = np.asarray(u, dtype=np.float32)
    Bsz, L, dm = h.shape
    ones = np.ones((dm,), dtype=np.float32)
    caches, stats = [], []
    for li, prep in enumerate(preps):
        xin = rmsnorm_fixed_order(h.reshape(Bsz * L, dm), ones).reshape(Bsz, L, dm)
        out, r, cache, st = layer_prefill(prep, shape, xin, mode, None if qps is None else qps[li],
                                          collect=qstats is not None, scan=scan)
        if qstats is not None:
            for pt in QS.POINTS:
                QS.accumulate(qstats[li], pt, r["qstats"][pt])
        h = h + out
        caches.append(cache)
        stats.append(st)
    return h, caches, stats


def stack_decode(preps, shape, u_t, caches, mode="dynamic", qps=None, state_fmts=None):
    """One decode step through the stack; returns (h_t [Bsz, d_model], new caches).

    ``state_fmts``: one (bits, shift) per layer for narrow state caches."""
    h = np.asarray(u_t, dtype=np.float32)
    dm = h.shape[-1]
    ones = np.ones((dm,), dtype=np.float32)
    new_caches = []
    for li, prep in enumerate(preps):
        xin = rmsnorm_fixed_order(h, ones)
        out, _, cache, _ = layer_decode(prep, shape, xin, caches[li], mode,
                                        None if qps is None else qps[li],
                                        None if state_fmts is None else state_fmts[li])
        h = h + out
        new_caches.append(cache)
    return h, new_caches


def qparams_from_stats(st: Stats) -> QParams:
    """Convert observed maxima to static (scoe, sshift) pairs and exponents."""
    def coef(amax):
        c = 127.0 / float(amax) if amax > 0 else 1.0
        m, e = np.frexp(c)                     # c = m * 2^e, m in [0.5, 1)
        sshift = 15 - int(e)                   # c * 2^sshift = m * 2^15 in [2^14, 2^15)
        scoe = int(np.rint(m * 2.0 ** 15))
        return scoe, sshift
    s0, h0 = coef(st.amax_u)
    s1, h1 = coef(st.amax_g)
    p = (pot_f32(st.amax_xbc),) + tuple(pot_q16(m) for m in st.amax_q16)
    return QParams(scoe=(s0, s1), sshift=(h0, h1), p=p)


def calibrate_stack(preps, shape, calib_inputs, scan=None):
    """Dynamic-mode passes over the calibration inputs; returns per-layer QParams
    and the maxima they come from.  ``scan`` as in layer_prefill."""
    acc = [Stats() for _ in preps]
    for u in calib_inputs:
        _, _, stats = stack_prefill(preps, shape, u, "dynamic", scan=scan)
        for a, st in zip(acc, stats):
            a.update(st)
    return [qparams_from_stats(a) for a in acc], acc
