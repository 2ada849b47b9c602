"""Device-memory owners around the C-ABI: one mixer layer, and pre-norm stacks.

These classes allocate torch device tensors (weights, caches, workspaces) and
call libfm.so; they compute nothing themselves.
"""
import ctypes

import numpy as np
import torch

from . import binding as B
from .configs import LayerShape


def _dev(a, dtype=None, device="cuda"):
    t = torch.as_tensor(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device).contiguous()


class GraphHeld(RuntimeError):
    """A buffer a captured graph points at would be reallocated."""


class WorkspacePool:
    """One device workspace shared by layers that run one call at a time.

    While a captured graph holds the pool (``holds`` > 0) it never regrows:
    the graph's kernels keep the current buffer's address."""

    def __init__(self, device="cuda"):
        self.device = device
        self.t = None
        self.holds = 0

    def get(self, need):
        if self.t is None or self.t.numel() < need:
            if self.holds:
                raise GraphHeld(f"workspace of {0 if self.t is None else self.t.numel()} bytes "
                                f"would grow to {need} while a captured graph uses it")
            self.t = None  # release before growing
            self.t = B.workspace(need, self.device)
        return self.t


class Mamba2Layer:
    """One quantized mixer layer with prepared weights, a workspace and a cache."""

    def __init__(self, shape: LayerShape, params: dict, mode: str = "dynamic",
                 prenorm_residual: bool = False, device="cuda", stream=None, ws_pool=None):
        s = shape
        self.shape = s
        self.device = device
        self.desc = B.LayerDesc(s.d_model, s.d_inner, s.nheads, s.headdim, s.dstate, s.d_conv,
                                B.STATIC if mode == "static" else B.DYNAMIC,
                                1 if prenorm_residual else 0)
        self.static = None
        f32 = torch.float32
        w_in = _dev(params["w_in"], f32, device)
        w_out = _dev(params["w_out"], f32, device)
        conv_w = _dev(params["conv_w"], f32, device)
        conv_b = _dev(params["conv_b"], f32, device)
        A = _dev(params["A"], f32, device)
        D = _dev(params["D"], f32, device)
        ch, dip, H = s.conv_ch, s.d_in_proj, s.nheads
        t = {}
        t["w_in_q"] = torch.empty((dip, s.d_model), dtype=torch.int8, device=device)
        t["s_w_in"] = torch.empty(1, dtype=f32, device=device)
        t["w_out_q"] = torch.empty((s.d_model, s.d_inner), dtype=torch.int8, device=device)
        t["s_w_out"] = torch.empty(1, dtype=f32, device=device)
        t["conv_w_q"] = torch.empty((ch, 4), dtype=torch.int8, device=device)
        t["conv_p_w"] = torch.empty(ch, dtype=torch.int32, device=device)
        t["conv_b_q16"] = torch.empty(ch, dtype=torch.int32, device=device)
        t["a_q16"] = torch.empty(H, dtype=torch.int32, device=device)
        t["d_q16"] = torch.empty(H, dtype=torch.int32, device=device)
        t["dt_bias"] = _dev(params["dt_bias"], f32, device)
        t["norm_w"] = _dev(params["norm_w"], f32, device)
        ws = B.workspace(B.lib.fm_prepare_layer_workspace_size(ctypes.byref(self.desc)), device)
        B._check(B.lib.fm_prepare_layer(
            ctypes.byref(self.desc), w_in.data_ptr(), w_out.data_ptr(), conv_w.data_ptr(),
            conv_b.data_ptr(), A.data_ptr(), D.data_ptr(), t["w_in_q"].data_ptr(),
            t["s_w_in"].data_ptr(), t["w_out_q"].data_ptr(), t["s_w_out"].data_ptr(),
            t["conv_w_q"].data_ptr(), t["conv_p_w"].data_ptr(), t["conv_b_q16"].data_ptr(),
            t["a_q16"].data_ptr(), t["d_q16"].data_ptr(), ws.data_ptr(), ws.numel(),
            B._stream(stream)))
        self.t = t
        self.weights = B.LayerWeights(*(t[n].data_ptr() for n in (
            "w_in_q", "s_w_in", "w_out_q", "s_w_out", "conv_w_q", "conv_p_w", "conv_b_q16",
            "dt_bias", "a_q16", "d_q16", "norm_w")))
        self.qp = torch.zeros(B.QPARAMS_BYTES, dtype=torch.uint8, device=device)
        self._pool = ws_pool
        self._ws = None
        self._ws_key = None
        self.cache = None
        self.ncache = None  # narrow state cache (narrow_state), used by decode when set
        self.holds = 0      # captured graphs pointing at this layer's caches / workspace

    def _check_not_held(self, what):
        if self.holds:
            raise GraphHeld(f"{what} would replace buffers a captured graph uses")

    # ------------------------------------------------------------ memory
    def workspace_for(self, batch, length, ssd=False):
        size = B.lib.fm_mamba2_layer_workspace_size_ssd if ssd else \
            B.lib.fm_mamba2_layer_workspace_size
        need = size(ctypes.byref(self.desc), batch, length)
        if self._pool is not None:
            self._ws = self._pool.get(need)
        elif self._ws is None or self._ws.numel() < need:
            self._check_not_held("growing the workspace")
            self._ws = B.workspace(need, self.device)
        self._ws_key = (batch, length)
        return self._ws

    def alloc_cache(self, batch):
        self._check_not_held("a new cache")
        s = self.shape
        self.cache_t = {
            "conv_state": torch.zeros((batch, s.conv_ch, 3), dtype=torch.int8, device=self.device),
            "ssm_state": torch.zeros((batch, s.nheads, s.headdim, s.dstate), dtype=torch.int32,
                                     device=self.device),
            "p": torch.zeros(4, dtype=torch.int32, device=self.device),
        }
        self.cache = B.Cache(self.cache_t["conv_state"].data_ptr(),
                             self.cache_t["ssm_state"].data_ptr(), self.cache_t["p"].data_ptr())
        return self.cache

    def narrow_state(self, bits, shift=None, headroom=1):
        """Convert the cache's int32 SSM state (as the last prefill left it) to
        `bits`-bit codes on the grid 2^shift; later decode calls use them.
        shift None: the smallest that holds 2^headroom times the current
        largest |state| unclipped.  Returns the shift."""
        self._check_not_held("narrowing the state")
        st = self.cache_t["ssm_state"]
        if shift is None:
            amax = torch.zeros(1, dtype=torch.int32, device=self.device)
            B.fm_state_absmax(st, amax)
            shift = B.fm_state_shift_for(int(amax.item()) & 0xFFFFFFFF, bits, headroom)
        codes = torch.empty(B.lib.fm_state_narrow_bytes(st.numel(), bits), dtype=torch.uint8,
                            device=self.device)
        B.fm_state_narrow(st, bits, shift, codes)
        self.cache_t["ssm_codes"] = codes
        self.ncache = B.CacheNarrow(self.cache_t["conv_state"].data_ptr(), codes.data_ptr(),
                                    self.cache_t["p"].data_ptr(), bits, shift)
        return shift

    def wide_state(self):
        """The narrow cache's state as int32 values c * 2^shift (a new tensor)."""
        st = self.cache_t["ssm_state"]
        out = torch.empty_like(st)
        B.fm_state_widen(self.cache_t["ssm_codes"], self.ncache.state_bits,
                         self.ncache.state_shift, out)
        return out

    def set_static(self, sp: "B.StaticParams"):
        self.static = sp
        self.desc.mode = B.STATIC

    def set_dynamic(self):
        self.desc.mode = B.DYNAMIC

    def reset_stats(self):
        self.qp.zero_()

    def qparams(self) -> "B.QParams":
        return B.qparams_from_device(self.qp)

    # ------------------------------------------------------------ calls
    def prefill(self, u, out=None, with_cache=True, stream=None, scan="sequential", opts=None):
        """u [batch, len, d_model] float32 device tensor -> out (same shape).
        scan "ssd": the chunked scan variant (fm_mamba2_layer_prefill_ssd);
        opts: a binding.LayerOpts for this call (binding.layer_opts) or None."""
        batch, length, dm = u.shape
        if out is None:
            out = torch.empty_like(u)
        ssd = scan == "ssd"
        if not ssd and scan != "sequential":
            raise ValueError(f"scan {scan!r}: 'sequential' or 'ssd'")
        ws = self.workspace_for(batch, length, ssd)
        cache = None
        if with_cache:
            if self.ncache is not None:  # a graph stepping the narrow codes would go stale
                self._check_not_held("a prefill over a narrow state")
            if self.cache is None or self.cache_t["ssm_state"].shape[0] != batch:
                self.alloc_cache(batch)
            self.ncache = None  # the prefill writes the int32 state
            cache = ctypes.byref(self.cache)
        sp = ctypes.byref(self.static) if self.static is not None else None
        fn = B.lib.fm_mamba2_layer_prefill_ssd if ssd else B.lib.fm_mamba2_layer_prefill
        B._check(fn(
            ctypes.byref(self.desc), ctypes.byref(self.weights), sp, u.data_ptr(), batch, length,
            out.data_ptr(), cache, self.qp.data_ptr(), B.opts_ref(opts), ws.data_ptr(),
            ws.numel(), B._stream(stream)))
        return out

    def decode(self, u_t, out=None, stream=None, opts=None):
        """u_t [batch, d_model] -> out_t, advancing the cache by one token."""
        batch, dm = u_t.shape
        if out is None:
            out = torch.empty_like(u_t)
        ws = self.workspace_for(batch, 1)
        sp = ctypes.byref(self.static) if self.static is not None else None
        if self.ncache is not None:
            B._check(B.lib.fm_mamba2_layer_decode_narrow(
                ctypes.byref(self.desc), ctypes.byref(self.weights), sp, u_t.data_ptr(), batch,
                ctypes.byref(self.ncache), out.data_ptr(), self.qp.data_ptr(),
                B.opts_ref(opts), ws.data_ptr(), ws.numel(), B._stream(stream)))
            return out
        B._check(B.lib.fm_mamba2_layer_decode(
            ctypes.byref(self.desc), ctypes.byref(self.weights), sp, u_t.data_ptr(), batch,
            ctypes.byref(self.cache), out.data_ptr(), self.qp.data_ptr(), B.opts_ref(opts),
            ws.data_ptr(), ws.numel(), B._stream(stream)))
        return out

    def taps(self, batch, length):
        t = B.LayerTaps()
        B._check(B.lib.fm_mamba2_layer_taps(ctypes.byref(self.desc), batch, length,
                                            ctypes.byref(t)))
        return t

    def tap(self, name, dtype, shape):
        """View of an intermediate the last call left in the workspace."""
        batch, length = self._ws_key
        off = getattr(self.taps(batch, length), name)
        n = int(np.prod(shape))
        itemsize = torch.tensor([], dtype=dtype).element_size()
        raw = self._ws[off:off + n * itemsize]
        return raw.view(dtype).view(*shape)


class Mamba2Stack:
    """Pre-norm residual stack: h <- h + layer(RMSNorm(h)) per layer."""

    def __init__(self, shape: LayerShape, params_list, mode="dynamic", device="cuda"):
        """``params_list``: any iterable of parameter dicts (a generator keeps only one
        layer's float32 weights on the host at a time)."""
        self.pool = WorkspacePool(device)
        self.layers = [Mamba2Layer(shape, p, mode, prenorm_residual=True, device=device,
                                   ws_pool=self.pool)
                       for p in params_list]
        self.shape = shape

    def prefill(self, u, with_cache=True, stream=None, quant_stats=None, layer_opts=None,
                bufs=None):
        """``quant_stats``: optional list of device fm_quant_stats buffers, one per
        layer (binding.quant_stats_buffer), into which each layer adds the
        statistics of its quantization points.  ``layer_opts``: optional list of
        per-layer binding.LayerOpts (taking precedence over quant_stats).
        ``bufs``: two tensors shaped like u for the residual stream (allocated
        if None); the result is one of them."""
        h = u.contiguous()
        if bufs is None:
            bufs = [torch.empty_like(h), torch.empty_like(h)]
        for i, layer in enumerate(self.layers):
            nxt = bufs[i % 2]
            if layer_opts is not None:
                opts = layer_opts[i]
            else:
                opts = None if quant_stats is None else B.layer_opts(quant_stats=quant_stats[i])
            layer.prefill(h, out=nxt, with_cache=with_cache, stream=stream, opts=opts)
            h = nxt
        return h

    def decode(self, u_t, stream=None):
        h = u_t.contiguous()
        bufs = [torch.empty_like(h), torch.empty_like(h)]
        for i, layer in enumerate(self.layers):
            nxt = bufs[i % 2]
            layer.decode(h, out=nxt, stream=stream)
            h = nxt
        return h

    def narrow_states(self, bits, headroom=1):
        """Every layer's cache to `bits`-bit codes (Mamba2Layer.narrow_state); the shifts."""
        return [layer.narrow_state(bits, None, headroom) for layer in self.layers]

    def calibrate(self, inputs):
        """Dynamic passes over `inputs` (list of [B, L, dm] device tensors), then static."""
        for layer in self.layers:
            layer.set_dynamic()
            layer.static = None
            layer.reset_stats()
        for u in inputs:
            self.prefill(u, with_cache=False)
        for layer in self.layers:
            layer.set_static(B.fm_qparams_from_stats(layer.qparams()))


class DecodeGraph:
    """One decode step of a stack (every layer's launches) captured as a HIP graph.

    The library neither allocates nor synchronizes inside a call and clears its
    scratch words with a kernel, so the whole step is capturable.  ``step``
    copies the input into the graph's fixed input buffer and replays; the
    returned tensor is the graph's output buffer (the next replay overwrites
    it).  Capture records work without running it, so the caches are not
    advanced by building the graph; the stack's workspace must already be
    sized (any earlier prefill or decode call on it does that).

    The graph's kernels hold raw addresses of the shared workspace and of every
    layer's caches.  While the graph is open it keeps references to those
    tensors and holds the pool and the layers: a call that would replace one
    (a prefill with another batch or a larger workspace, narrowing the state)
    raises GraphHeld instead.  ``close()`` (or leaving a ``with`` block) lets
    them go; ``step`` also checks the recorded addresses and refuses to replay
    a closed graph."""

    def __init__(self, stack: Mamba2Stack, batch: int, device="cuda"):
        self.stack = stack
        self.x = torch.zeros((batch, stack.shape.d_model), dtype=torch.float32, device=device)
        for layer in stack.layers:  # size the shared workspace outside the capture
            layer.workspace_for(batch, 1)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.out = stack.decode(self.x)
        self._held = self._buffers()
        self._ptrs = tuple(t.data_ptr() for t in self._held)
        stack.pool.holds += 1
        for layer in stack.layers:
            layer.holds += 1
        self.open = True

    def _buffers(self):
        ts = [self.stack.pool.t]
        for layer in self.stack.layers:
            ts += [layer.cache_t[k] for k in ("conv_state", "ssm_state", "p")]
            if layer.ncache is not None:
                ts.append(layer.cache_t["ssm_codes"])
        return ts

    def close(self):
        if self.open:
            self.open = False
            self.stack.pool.holds -= 1
            for layer in self.stack.layers:
                layer.holds -= 1
            self._held = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def step(self, x):
        if not self.open:
            raise GraphHeld("the decode graph is closed")
        if tuple(t.data_ptr() for t in self._buffers()) != self._ptrs:
            raise GraphHeld("a buffer the decode graph uses was replaced")
        self.x.copy_(x)
        self.graph.replay()
        return self.out
