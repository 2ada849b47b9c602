"""ctypes binding of libfm.so (include/fm.h): argument marshalling only.

Every function here has the name of a C entry point and forwards torch
tensors' device pointers and sizes to it; every step of the method runs in the
library's HIP kernels.  The library is loaded from this package's directory;
if it is missing the import fails loudly — there is no fallback path.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfm.so")

FM_OK, FM_ERR_NULL, FM_ERR_SHAPE, FM_ERR_MODE, FM_ERR_WORKSPACE, FM_ERR_HIP = range(6)
DYNAMIC, STATIC = 0, 1


class FmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"fm status {status}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m quantized_state_space_fwht_amd.build` (no fallback exists)")
    return ctypes.CDLL(LIB_PATH)


lib = _load()

_c_i64, _c_i32, _c_sz, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p


class LayerDesc(ctypes.Structure):
    _fields_ = [("d_model", _c_i64), ("d_inner", _c_i64), ("nheads", _c_i64),
                ("headdim", _c_i64), ("dstate", _c_i64), ("d_conv", _c_i64),
                ("mode", _c_i32), ("prenorm_residual", _c_i32)]


class StaticParams(ctypes.Structure):
    _fields_ = [("scoe", _c_i32 * 2), ("sshift", _c_i32 * 2), ("p", _c_i32 * 4)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w_in_q", "s_w_in", "w_out_q", "s_w_out", "conv_w_q",
                                   "conv_p_w", "conv_b_q16", "dt_bias", "a_q16", "d_q16",
                                   "norm_w")]


class QParams(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float * 2), ("p", _c_i32 * 4),
                ("stat_amax", ctypes.c_float * 3), ("stat_amax_q16", _c_i32 * 3),
                ("reserved", _c_i32 * 4)]


class Cache(ctypes.Structure):
    _fields_ = [("conv_state", _vp), ("ssm_state", _vp), ("p", _vp)]


class CacheNarrow(ctypes.Structure):
    _fields_ = [("conv_state", _vp), ("ssm_state", _vp), ("p", _vp), ("state_bits", _c_i32),
                ("state_shift", _c_i32)]


LAYER_EVENTS = 7  # FM_LAYER_EVENTS: stage boundaries of a layer call
STAGES = ("in_quant", "in_proj", "conv", "scan", "gate_quant", "out_proj")


class LayerOpts(ctypes.Structure):
    _fields_ = [("keep_intermediates", _c_i32), ("reserved", _c_i32), ("quant_stats", _vp),
                ("stage_events", ctypes.POINTER(_vp))]


def layer_opts(keep=False, quant_stats=None, events=None):
    """A per-call fm_layer_opts, or None when every option is off.

    quant_stats: a device fm_quant_stats buffer (quant_stats_buffer);
    events: LAYER_EVENTS torch.cuda.Event or None entries (stage boundaries)."""
    if not keep and quant_stats is None and events is None:
        return None
    o = LayerOpts()
    o.keep_intermediates = 1 if keep else 0
    o.quant_stats = None if quant_stats is None else quant_stats.data_ptr()
    if events is not None:
        if len(events) != LAYER_EVENTS:
            raise ValueError(f"events: {LAYER_EVENTS} entries")
        arr = (_vp * LAYER_EVENTS)(*[None if e is None else e.cuda_event for e in events])
        o._events = arr  # keep the array alive with the struct
        o.stage_events = ctypes.cast(arr, ctypes.POINTER(_vp))
    return o


def opts_ref(o):
    return None if o is None else ctypes.byref(o)


class LayerTaps(ctypes.Structure):
    _fields_ = [(n, _c_sz) for n in ("u_q", "v", "xbc_q", "x_q", "b_q", "c_q", "y", "g_q",
                                     "normed", "dt", "da")]


QPARAMS_BYTES = ctypes.sizeof(QParams)

_SIGS = {
    "fm_abi_version": (ctypes.c_int, []),
    "fm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fm_last_error": (ctypes.c_char_p, []),
    "fm_hadamard_quant_workspace_size": (_c_sz, [_c_i64, _c_i64]),
    "fm_hadamard_quant": (ctypes.c_int, [_vp, _c_i64, _c_i64, ctypes.c_int, _c_i32, _c_i32, _vp,
                                         _vp, _vp, _vp, _c_sz, _vp]),
    "fm_w8a8_gemm": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp]),
    "fm_conv1d_pot_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i64]),
    "fm_conv1d_pot": (ctypes.c_int, [_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp,
                                     ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _c_sz, _vp]),
    "fm_ssm_scan_pot_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_i64]),
    "fm_ssm_scan_pot": (ctypes.c_int, [_vp, _vp, _vp, _vp, _c_i64, _vp, _vp, _vp, _vp, _c_i64,
                                       _c_i64, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _c_sz, _vp]),
    "fm_nau_eval": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _c_i64, _vp]),
    "fm_gate_norm_quant_workspace_size": (_c_sz, [_c_i64, _c_i64]),
    "fm_gate_norm_quant": (ctypes.c_int, [_vp, _vp, _c_i64, _vp, _vp, _c_i64, _c_i64,
                                          ctypes.c_int, _c_i32, _c_i32, _vp, _vp, _vp, _vp, _vp,
                                          _c_sz, _vp]),
    "fm_prepare_layer_workspace_size": (_c_sz, [ctypes.POINTER(LayerDesc)]),
    "fm_prepare_layer": (ctypes.c_int, [ctypes.POINTER(LayerDesc)] + [_vp] * 15 + [_vp, _c_sz,
                                                                                 _vp]),
    "fm_mamba2_layer_workspace_size": (_c_sz, [ctypes.POINTER(LayerDesc), _c_i64, _c_i64]),
    "fm_mamba2_layer_prefill": (ctypes.c_int, [ctypes.POINTER(LayerDesc),
                                               ctypes.POINTER(LayerWeights),
                                               ctypes.POINTER(StaticParams), _vp, _c_i64, _c_i64,
                                               _vp, ctypes.POINTER(Cache), _vp,
                                               ctypes.POINTER(LayerOpts), _vp, _c_sz, _vp]),
    "fm_mamba2_layer_decode": (ctypes.c_int, [ctypes.POINTER(LayerDesc),
                                              ctypes.POINTER(LayerWeights),
                                              ctypes.POINTER(StaticParams), _vp, _c_i64,
                                              ctypes.POINTER(Cache), _vp, _vp,
                                              ctypes.POINTER(LayerOpts), _vp, _c_sz, _vp]),
    "fm_mamba2_layer_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(LayerDesc),
                                                      ctypes.POINTER(LayerWeights),
                                                      ctypes.POINTER(StaticParams), _vp, _c_i64,
                                                      ctypes.POINTER(Cache), _vp, _vp,
                                                      ctypes.POINTER(LayerOpts), _vp]),
    "fm_mamba2_layer_taps": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _c_i64, _c_i64,
                                            ctypes.POINTER(LayerTaps)]),
    "fm_nau_eval_knots": (ctypes.c_int, [_c_i32, _vp, _vp, _vp, _c_i64, _vp]),
    "fm_quant_per_tensor_workspace_size": (_c_sz, []),
    "fm_quant_per_tensor": (ctypes.c_int, [_vp, _c_i64, _vp, _vp, _vp, _c_sz, _vp]),
    "fm_smooth_scales_workspace_size": (_c_sz, [_c_i64]),
    "fm_smooth_scales": (ctypes.c_int, [_vp, _c_i64, _vp, _c_i64, _c_i64, _vp, _vp, _c_sz, _vp]),
    "fm_scale_columns": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _c_i32, _vp, _vp]),
    "fm_qparams_from_stats": (ctypes.c_int, [ctypes.POINTER(QParams),
                                             ctypes.POINTER(StaticParams)]),
    "fm_ssm_scan_ssd_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64]),
    "fm_ssm_scan_ssd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _c_i64, _vp, _vp, _vp, _vp, _c_i64,
                                       _c_i64, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _c_sz, _vp]),
    "fm_mamba2_layer_workspace_size_ssd": (_c_sz, [ctypes.POINTER(LayerDesc), _c_i64, _c_i64]),
    "fm_mamba2_layer_prefill_ssd": (ctypes.c_int, [ctypes.POINTER(LayerDesc),
                                                   ctypes.POINTER(LayerWeights),
                                                   ctypes.POINTER(StaticParams), _vp, _c_i64,
                                                   _c_i64, _vp, ctypes.POINTER(Cache), _vp,
                                                   ctypes.POINTER(LayerOpts), _vp, _c_sz, _vp]),
    "fm_state_narrow_bytes": (_c_sz, [_c_i64, _c_i32]),
    "fm_state_narrow": (ctypes.c_int, [_vp, _c_i64, _c_i32, _c_i32, _vp, _vp]),
    "fm_state_widen": (ctypes.c_int, [_vp, _c_i64, _c_i32, _c_i32, _vp, _vp]),
    "fm_state_absmax": (ctypes.c_int, [_vp, _c_i64, _vp, _vp]),
    "fm_state_shift_for": (ctypes.c_int, [ctypes.c_uint32, _c_i32, _c_i32,
                                          ctypes.POINTER(_c_i32)]),
    "fm_mamba2_layer_decode_narrow": (ctypes.c_int, [ctypes.POINTER(LayerDesc),
                                                     ctypes.POINTER(LayerWeights),
                                                     ctypes.POINTER(StaticParams), _vp, _c_i64,
                                                     ctypes.POINTER(CacheNarrow), _vp, _vp,
                                                     ctypes.POINTER(LayerOpts), _vp, _c_sz, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


def _check(status):
    if status != FM_OK:
        raise FmError(status, lib.fm_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous"
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def workspace(nbytes, device="cuda"):
    """A 256-byte aligned device buffer (torch's allocator aligns to >= 512 bytes)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- step calls
def fm_hadamard_quant(x, mode, scoe, sshift, q, scale_out, amax_stats=None, ws=None, stream=None):
    rows, k = x.shape
    if ws is None and mode == DYNAMIC:
        ws = workspace(lib.fm_hadamard_quant_workspace_size(rows, k), x.device)
    _check(lib.fm_hadamard_quant(_ptr(x), rows, k, mode, scoe, sshift, _ptr(q), _ptr(scale_out),
                                 _ptr(amax_stats), _ptr(ws), 0 if ws is None else ws.numel(),
                                 _stream(stream)))


def fm_nau_eval_knots(fn, knots_q30, x, y, stream=None):
    """knots_q30: nine Q.30 integers (host, any sequence)."""
    arr = (ctypes.c_int64 * 9)(*[int(v) for v in knots_q30])
    _check(lib.fm_nau_eval_knots(fn, ctypes.cast(arr, ctypes.c_void_p), _ptr(x), _ptr(y),
                                 x.numel(), _stream(stream)))


def fm_state_narrow(state, bits, shift, codes, stream=None):
    """int32 state tensor -> codes (a uint8 device tensor of fm_state_narrow_bytes bytes)."""
    n = state.numel()
    if codes.numel() * codes.element_size() < lib.fm_state_narrow_bytes(n, bits):
        raise ValueError("codes buffer too small")
    _check(lib.fm_state_narrow(_ptr(state), n, bits, shift, _ptr(codes), _stream(stream)))


def fm_state_widen(codes, bits, shift, state, stream=None):
    n = state.numel()
    if codes.numel() * codes.element_size() < lib.fm_state_narrow_bytes(n, bits):
        raise ValueError("codes buffer too small")
    _check(lib.fm_state_widen(_ptr(codes), n, bits, shift, _ptr(state), _stream(stream)))


def fm_state_absmax(state, amax, stream=None):
    """amax: one-element int32/uint32 device tensor, max-accumulated."""
    _check(lib.fm_state_absmax(_ptr(state), state.numel(), _ptr(amax), _stream(stream)))


def fm_state_shift_for(amax, bits, headroom=1):
    """The narrow-state shift for a largest |state| of amax (host call)."""
    out = _c_i32()
    _check(lib.fm_state_shift_for(int(amax) & 0xFFFFFFFF, bits, headroom, ctypes.byref(out)))
    return out.value


def fm_quant_per_tensor(x, q, scale_out, ws=None, stream=None):
    if ws is None:
        ws = workspace(lib.fm_quant_per_tensor_workspace_size(), x.device)
    _check(lib.fm_quant_per_tensor(_ptr(x), x.numel(), _ptr(q), _ptr(scale_out), _ptr(ws),
                                   ws.numel(), _stream(stream)))


def fm_smooth_scales(x, w, s, ws=None, stream=None):
    rows, k = x.shape
    n = w.shape[0]
    if ws is None:
        ws = workspace(lib.fm_smooth_scales_workspace_size(k), x.device)
    _check(lib.fm_smooth_scales(_ptr(x), rows, _ptr(w), n, k, _ptr(s), _ptr(ws), ws.numel(),
                                _stream(stream)))


def fm_scale_columns(x, s, divide, out, stream=None):
    rows, k = x.shape
    _check(lib.fm_scale_columns(_ptr(x), rows, k, _ptr(s), 1 if divide else 0, _ptr(out),
                                _stream(stream)))


def fm_w8a8_gemm(a, b, scale_a, scale_b, acc=None, out=None, stream=None):
    m, k = a.shape
    n = b.shape[0]
    _check(lib.fm_w8a8_gemm(_ptr(a), _ptr(b), m, n, k, _ptr(scale_a), _ptr(scale_b), _ptr(acc),
                            _ptr(out), _stream(stream)))


def fm_conv1d_pot(xbc, row_stride, batch, length, d_inner, dstate, w_q, p_w, b_q16, mode,
                  p_fixed, state_in, state_out, xbc_q, x_out, b_out, c_out, p_out,
                  amax_stats=None, ws=None, stream=None):
    if ws is None:
        ws = workspace(lib.fm_conv1d_pot_workspace_size(batch, length, d_inner, dstate),
                       xbc.device)
    _check(lib.fm_conv1d_pot(xbc.data_ptr(), row_stride, batch, length, d_inner, dstate,
                             _ptr(w_q), _ptr(p_w), _ptr(b_q16), mode, _ptr(p_fixed),
                             _ptr(state_in), _ptr(state_out), _ptr(xbc_q), _ptr(x_out),
                             _ptr(b_out), _ptr(c_out), _ptr(p_out), _ptr(amax_stats), _ptr(ws),
                             ws.numel(), _stream(stream)))


def fm_ssm_scan_pot(x, bm, cm, dt_raw, dt_row_stride, dt_bias, a_q16, d_q16, p, batch, length,
                    nheads, headdim, dstate, state_in, state_out, y, dt_out=None, da_out=None,
                    ws=None, stream=None):
    if ws is None:
        ws = workspace(lib.fm_ssm_scan_pot_workspace_size(batch, length, dstate), y.device)
    _check(lib.fm_ssm_scan_pot(_ptr(x), _ptr(bm), _ptr(cm), dt_raw.data_ptr(), dt_row_stride,
                               _ptr(dt_bias), _ptr(a_q16), _ptr(d_q16), _ptr(p), batch, length,
                               nheads, headdim, dstate, _ptr(state_in), _ptr(state_out), _ptr(y),
                               _ptr(dt_out), _ptr(da_out), _ptr(ws), ws.numel(),
                               _stream(stream)))


def fm_ssm_scan_ssd(x, bm, cm, dt_raw, dt_row_stride, dt_bias, a_q16, d_q16, p, batch, length,
                    nheads, headdim, dstate, state_in, state_out, y, dt_out=None, da_out=None,
                    ws=None, stream=None):
    """The chunked variant of fm_ssm_scan_pot (same arguments)."""
    if ws is None:
        ws = workspace(lib.fm_ssm_scan_ssd_workspace_size(batch, length, nheads, headdim,
                                                          dstate), y.device)
    _check(lib.fm_ssm_scan_ssd(_ptr(x), _ptr(bm), _ptr(cm), dt_raw.data_ptr(), dt_row_stride,
                               _ptr(dt_bias), _ptr(a_q16), _ptr(d_q16), _ptr(p), batch, length,
                               nheads, headdim, dstate, _ptr(state_in), _ptr(state_out), _ptr(y),
                               _ptr(dt_out), _ptr(da_out), _ptr(ws), ws.numel(),
                               _stream(stream)))


def fm_gate_norm_quant(y, z, z_row_stride, p, norm_w, rows, d_inner, mode, scoe, sshift, q,
                       scale_out, amax_stats=None, normed_out=None, ws=None, stream=None):
    if ws is None:
        ws = workspace(lib.fm_gate_norm_quant_workspace_size(rows, d_inner), y.device)
    _check(lib.fm_gate_norm_quant(_ptr(y), z.data_ptr(), z_row_stride, _ptr(p), _ptr(norm_w),
                                  rows, d_inner, mode, scoe, sshift, _ptr(q), _ptr(scale_out),
                                  _ptr(amax_stats), _ptr(normed_out), _ptr(ws), ws.numel(),
                                  _stream(stream)))


NAU_EXP, NAU_SOFTPLUS, NAU_SILU = 0, 1, 2


def fm_nau_eval(fn, x, y, stream=None):
    _check(lib.fm_nau_eval(fn, _ptr(x), _ptr(y), x.numel(), _stream(stream)))


def fm_qparams_from_stats(qp_host: QParams) -> StaticParams:
    sp = StaticParams()
    _check(lib.fm_qparams_from_stats(ctypes.byref(qp_host), ctypes.byref(sp)))
    return sp


def qparams_from_device(qp_dev) -> QParams:
    """Copy a device fm_qparams block to a host QParams (synchronizes)."""
    raw = qp_dev.cpu().numpy().tobytes()
    return QParams.from_buffer_copy(raw)


# quantization points of fm_quant_stats
QP_U, QP_G, QP_XBC, QP_X, QP_B, QP_C = range(6)
QP_NAMES = ("u", "g", "xbc", "x", "B", "C")


class QuantStats(ctypes.Structure):
    _fields_ = [("count", ctypes.c_ulonglong * 6), ("clipped", ctypes.c_ulonglong * 6),
                ("sq_err", ctypes.c_double * 6), ("sq_val", ctypes.c_double * 6)]


def quant_stats_buffer(device="cuda"):
    """A zeroed device fm_quant_stats (as a uint8 tensor)."""
    return torch.zeros(ctypes.sizeof(QuantStats), dtype=torch.uint8, device=device)


def quant_stats_from_device(buf) -> QuantStats:
    """Copy a device fm_quant_stats to the host (synchronizes)."""
    return QuantStats.from_buffer_copy(buf.cpu().numpy().tobytes())
