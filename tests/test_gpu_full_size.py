"""GPU parity at the full sizes of the workloads.

Every oracle input is seeded and synthetic, or the oracle's own result: what
the GPU computes is compared with the oracle, never fed to it.  Where the
oracle cannot follow a whole workload, it recomputes whole layers or whole
sequences at the real shapes (its C scan makes full-size layers affordable),
and the rest is checked by properties that hold at any size.

* m130m_layer (batch 1, L 2048): the prefill benchmark's own call (no
  intermediates kept), the whole layer in the oracle: output, state, conv
  window, scales and exponents bit for bit.  (The parity file compares every
  intermediate of the same layer as well.)
* m2p7b_stack (batch 4, L 4096, dynamic): the first three layers chained, every
  layer's output, caches and record bit for bit and every intermediate of
  layer 0; the 64-layer stack under batch-permutation equivariance (per-tensor
  maxima do not depend on the order of the rows, everything else is row- or
  sequence-local, so reversing the batch reverses the output bit for bit).
* m130m_stack_static (batch 8, L 2048): all 24 layers calibrated on the first
  four calibration sequences by both sides, every layer's maxima and static
  parameters equal; then one whole evaluation sequence through the 24 static
  layers, the stack output and every layer's caches bit for bit.  The stack
  calibrated on all 64 sequences: layer 0's maxima equal the oracle's over the
  64 sequences, and two properties on the evaluation batch (a sequence alone
  gives its row of the batch; a prefill continued by decode steps gives the
  longer prefill).
* m2p7b_decode (batch 16): layers 0 and 63 as one-layer graph-replayed decode
  stacks seeded by the workload's 1024-token prefill, which the oracle runs
  too; every step bit for bit with the int32 state and with 24- and 16-bit
  state codes; the 64-layer stack's graph replays equal its eager steps.
"""
import numpy as np
import pytest

import oracle as O
from oracle.scan_c import ssm_scan_pot_c
from quantized_state_space_fwht_amd import configs, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def B():
    from quantized_state_space_fwht_amd import binding
    return binding


def dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).cuda().contiguous()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_exact(got, want, what):
    got = np.asarray(got).astype(np.int64)
    want = np.asarray(want).astype(np.int64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[0]}: " \
                          f"gpu {got[tuple(bad[0])]} oracle {want[tuple(bad[0])]}"


def assert_same_float(got, want, what):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} differ, first at {bad[0]}: " \
                          f"gpu {got[tuple(bad[0])]!r} oracle {want[tuple(bad[0])]!r}"


def prenorm(u):
    dm = u.shape[-1]
    return O.rmsnorm_fixed_order(u.reshape(-1, dm), np.ones(dm, np.float32)).reshape(u.shape)


def check_caches_and_record(layer, cache_o, r, st_o):
    assert_exact(host(layer.cache_t["ssm_state"]), cache_o["ssm_state"], "ssm state")
    assert_exact(host(layer.cache_t["conv_state"]), cache_o["conv_state"], "conv window")
    assert_exact(host(layer.cache_t["p"]), cache_o["p"], "cached exponents")
    qp = layer.qparams()
    assert qp.scale[0] == r["s_u"] and qp.scale[1] == r["s_g"]
    assert tuple(qp.p) == tuple(r["p"])
    assert qp.stat_amax[0] == np.float32(st_o.amax_u)
    assert qp.stat_amax[2] == np.float32(st_o.amax_xbc)
    assert list(qp.stat_amax_q16) == list(st_o.amax_q16)


def check_intermediates(layer, r, T, s):
    g = lambda name, dt, shp: layer.tap(name, dt, shp).cpu().numpy()
    assert_exact(g("u_q", torch.int8, (T, s.d_model)), r["u_q"], "u_q")
    assert np.array_equal(g("v", torch.float32, (T, s.d_in_proj)), r["v"]), "in_proj output"
    assert_exact(g("xbc_q", torch.int8, (T, s.conv_ch)), r["xbc_q"], "xbc_q")
    assert_exact(g("x_q", torch.int8, (T, s.d_inner)), r["x_q"].reshape(T, -1), "x_q")
    assert_exact(g("b_q", torch.int8, (T, s.dstate)), r["B_q"].reshape(T, -1), "B_q")
    assert_exact(g("c_q", torch.int8, (T, s.dstate)), r["C_q"].reshape(T, -1), "C_q")
    assert_exact(g("dt", torch.int32, (T, s.nheads)), r["dt"].reshape(T, -1), "dt")
    assert_exact(g("da", torch.int32, (T, s.nheads)), r["dA"].reshape(T, -1), "dA")
    assert_exact(g("y", torch.int32, (T, s.d_inner)), r["y"].reshape(T, -1), "y")
    assert np.array_equal(g("normed", torch.float32, (T, s.d_inner)), r["normed"]), "normed"
    assert_exact(g("g_q", torch.int8, (T, s.d_inner)), r["g_q"], "g_q")


# ----------------------------------------------------------------- m130m_layer
def test_m130m_layer_full_size_as_benchmarked(B):
    from quantized_state_space_fwht_amd.runtime import Mamba2Layer
    w = configs.get("m130m_layer")
    s = w.shape
    params = synth.workload_params(w, 0)
    u = synth.workload_activations(w)
    out_o, r, cache_o, st_o = O.layer_prefill(O.prepare_layer(params), s, u,
                                              scan=ssm_scan_pot_c)
    layer = Mamba2Layer(s, params)
    ud = dev(u)
    out = torch.empty_like(ud)
    for _ in range(2):  # the benchmark's repeated calls on one layer and workspace
        layer.prefill(ud, out)
        assert_same_float(host(out), out_o, "layer output")
        check_caches_and_record(layer, cache_o, r, st_o)
        layer.reset_stats()


# ----------------------------------------------------------------- m2p7b_stack
def test_m2p7b_layer_ragged_rows_large_product(B):
    """A 2.7B pre-norm layer over 1 x 3228 rows: the in_proj product takes the
    large-product kernel (13 x 83 tiles of 256 x 128, over four per CU) with a
    partial last row tile, whose z columns go through the epilogue's SiLU one
    element at a time; bit-exact against the oracle."""
    from quantized_state_space_fwht_amd.runtime import Mamba2Layer
    w = configs.with_len(configs.get("m2p7b_stack"), batch=1, seqlen=3228)
    s = w.shape
    params = synth.workload_params(w, 0)
    u = synth.workload_activations(w)
    out_o, r, cache_o, st_o = O.layer_prefill(O.prepare_layer(params), s, prenorm(u),
                                              scan=ssm_scan_pot_c)
    layer = Mamba2Layer(s, params, prenorm_residual=True)
    h = layer.prefill(dev(u))
    assert_same_float(host(h), u + out_o, "layer output")
    check_caches_and_record(layer, cache_o, r, st_o)


def test_m2p7b_stack_first_layers_chained_full_size(B):
    """Layers 0, 1, 2 of the 2.7B stack at 4 x 4096, chained: the oracle runs the
    three layers itself (layer 0 on the input, each next layer on its own output)."""
    from quantized_state_space_fwht_amd.runtime import Mamba2Layer
    w = configs.get("m2p7b_stack")
    s = w.shape
    u = synth.workload_activations(w)
    T = w.batch * w.seqlen
    h_o = u
    h = dev(u)
    for l in range(3):
        params = synth.workload_params(w, l)
        out_o, r, cache_o, st_o = O.layer_prefill(O.prepare_layer(params), s, prenorm(h_o),
                                                  scan=ssm_scan_pot_c)
        h_o = h_o + out_o
        layer = Mamba2Layer(s, params, prenorm_residual=True)
        h = layer.prefill(h, opts=B.layer_opts(keep=(l == 0)))
        if l == 0:
            check_intermediates(layer, r, T, s)
        assert_same_float(host(h), h_o, f"layer {l} output")
        check_caches_and_record(layer, cache_o, r, st_o)
        del layer, r
        torch.cuda.empty_cache()


def test_m2p7b_stack_full_size_batch_permutation(B):
    """64 layers at 4 x 4096, dynamic: reversing the batch reverses the output."""
    from quantized_state_space_fwht_amd.runtime import Mamba2Stack
    w = configs.get("m2p7b_stack")
    stack = Mamba2Stack(w.shape, (synth.workload_params(w, l) for l in range(w.nlayers)))
    u = synth.workload_activations(w)
    h = host(stack.prefill(dev(u), with_cache=False))
    assert np.all(np.isfinite(h))
    h_rev = host(stack.prefill(dev(u[::-1]), with_cache=False))
    assert_same_float(h_rev, h[::-1], "reversed batch")


# ----------------------------------------------------------------- m130m_stack_static
def test_m130m_static_stack_calibrated_and_chained_full_size(B):
    """All 24 layers calibrated on the first four calibration sequences by both
    sides (each sequence whole, 1 x 2048), then one evaluation sequence through
    the 24 static layers."""
    from quantized_state_space_fwht_amd.runtime import Mamba2Stack
    w = configs.get("m130m_stack_static")
    s = w.shape
    params = [synth.workload_params(w, l) for l in range(w.nlayers)]
    preps = [O.prepare_layer(p) for p in params]
    calib = synth.calibration_sequences(w)[:4]
    qps_o, acc_o = O.calibrate_stack(preps, s, calib, scan=ssm_scan_pot_c)
    stack = Mamba2Stack(s, params)
    stack.calibrate([dev(c) for c in calib])
    for l, (layer, qo, ao) in enumerate(zip(stack.layers, qps_o, acc_o)):
        qp = layer.qparams()
        assert tuple(qp.stat_amax) == (np.float32(ao.amax_u), np.float32(ao.amax_g),
                                       np.float32(ao.amax_xbc)), f"layer {l} maxima"
        assert list(qp.stat_amax_q16) == list(ao.amax_q16), f"layer {l} Q.16 maxima"
        sp = layer.static
        assert (tuple(sp.scoe), tuple(sp.sshift), tuple(sp.p)) == (qo.scoe, qo.sshift, qo.p), \
            f"layer {l} static parameters"
    u = synth.eval_batch(w)
    h = host(stack.prefill(dev(u)))
    bsel = 5
    h_o, caches_o, _ = O.stack_prefill(preps, s, u[bsel:bsel + 1], "static", qps_o,
                                       scan=ssm_scan_pot_c)
    assert_same_float(h[bsel:bsel + 1], h_o, "stack output, one evaluation sequence")
    for l, (layer, co) in enumerate(zip(stack.layers, caches_o)):
        assert_exact(host(layer.cache_t["ssm_state"])[bsel], co["ssm_state"][0], f"layer {l} state")
        assert_exact(host(layer.cache_t["conv_state"])[bsel], co["conv_state"][0],
                     f"layer {l} conv window")


def test_m130m_static_stack_64_sequence_calibration_full_size(B):
    """The stack calibrated on all 64 sequences: layer 0's maxima equal the oracle's
    maximum over the 64 sequences (layer 0's input does not depend on the other
    layers); then properties of the static stack on the evaluation batch."""
    from quantized_state_space_fwht_amd.runtime import Mamba2Stack
    w = configs.get("m130m_stack_static")
    s = w.shape
    params = [synth.workload_params(w, l) for l in range(w.nlayers)]
    stack = Mamba2Stack(s, params)
    calib = synth.calibration_sequences(w)
    stack.calibrate([dev(c) for c in calib])
    prep0 = O.prepare_layer(params[0])
    acc = O.Stats()
    for c in calib:
        _, _, _, st = O.layer_prefill(prep0, s, prenorm(c), scan=ssm_scan_pot_c)
        acc.update(st)
    qp0 = stack.layers[0].qparams()
    assert tuple(qp0.stat_amax) == (np.float32(acc.amax_u), np.float32(acc.amax_g),
                                    np.float32(acc.amax_xbc))
    assert list(qp0.stat_amax_q16) == list(acc.amax_q16)
    # properties of the static stack on the evaluation batch
    u = synth.eval_batch(w)
    h = host(stack.prefill(dev(u)))
    assert np.all(np.isfinite(h))
    bsel = 5
    assert_same_float(host(stack.prefill(dev(u[bsel:bsel + 1]))), h[bsel:bsel + 1],
                      "a sequence alone")
    L0 = w.seqlen - 6
    stack.prefill(dev(u[:, :L0]))
    steps = [host(stack.decode(dev(u[:, t]))) for t in range(L0, w.seqlen)]
    assert_same_float(np.stack(steps, axis=1), h[:, L0:], "prefill continued by decode")


# ----------------------------------------------------------------- m2p7b_decode
@pytest.mark.parametrize("layer_idx", [0, 63])
def test_m2p7b_decode_layer_full_size(B, layer_idx):
    """One 2.7B layer at batch 16, graph-replayed as the decode benchmark runs its
    layers, seeded by the workload's 1024-token prefill (which the oracle runs
    too), then four decode steps on the workload's step inputs: with the int32
    state, and with 24- and 16-bit state codes on the shift the oracle picks."""
    from quantized_state_space_fwht_amd.runtime import DecodeGraph, Mamba2Stack
    w = configs.get("m2p7b_decode")
    s = w.shape
    K = 4
    params = synth.workload_params(w, layer_idx)
    u = synth.workload_activations(w)
    xs = [synth.decode_step_input(w, t) for t in range(K)]
    prep = O.prepare_layer(params)
    _, _, cache0, _ = O.layer_prefill(prep, s, prenorm(u), scan=ssm_scan_pot_c)
    stack = Mamba2Stack(s, [params])
    layer = stack.layers[0]
    for bits in (32, 24, 16):
        stack.prefill(dev(u))
        assert_exact(host(layer.cache_t["ssm_state"]), cache0["ssm_state"], "state after prefill")
        cache = dict(cache0)
        fmt = None
        if bits != 32:
            shift = O.state_shift_for(int(np.max(np.abs(cache0["ssm_state"]))), bits)
            assert layer.narrow_state(bits) == shift, f"{bits}-bit shift"
            fmt = (bits, shift)
            cache["ssm_state"] = O.narrow_state(cache0["ssm_state"], bits, shift)
        with DecodeGraph(stack, w.batch) as g:
            for t, x in enumerate(xs):
                out_o, _, cache, _ = O.layer_decode(prep, s, prenorm(x), cache, state_fmt=fmt)
                got = host(g.step(dev(x)))
                assert_same_float(got, x + out_o, f"layer {layer_idx} {bits}-bit step {t}")
                if bits == 32:
                    assert_exact(host(layer.cache_t["ssm_state"]), cache["ssm_state"],
                                 f"state step {t}")
                else:
                    assert_exact(host(layer.cache_t["ssm_codes"]),
                                 O.pack_state(cache["ssm_state"], bits), f"codes step {t}")
                assert_exact(host(layer.cache_t["conv_state"]), cache["conv_state"],
                             f"conv step {t}")


def test_m2p7b_decode_stack_graph_equals_eager(B):
    """The 64-layer decode stack: graph replays give the eager steps bit for bit."""
    from quantized_state_space_fwht_amd.runtime import DecodeGraph, Mamba2Stack
    w = configs.get("m2p7b_decode")
    stack = Mamba2Stack(w.shape, (synth.workload_params(w, l) for l in range(w.nlayers)))
    stack.prefill(dev(synth.workload_activations(w)))
    snap = [{k: v.clone() for k, v in layer.cache_t.items()} for layer in stack.layers]
    xs = [dev(synth.decode_step_input(w, t)) for t in range(3)]
    eager = [host(stack.decode(x)) for x in xs]
    for layer, c in zip(stack.layers, snap):
        for k, v in c.items():
            layer.cache_t[k].copy_(v)
    g = DecodeGraph(stack, w.batch)
    for t, x in enumerate(xs):
        assert_same_float(host(g.step(x)), eager[t], f"graph step {t}")
    assert np.all(np.isfinite(eager[-1]))
