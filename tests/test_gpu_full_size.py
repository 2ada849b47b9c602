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
* m2p7b_stack (batch 4, L 4096, dynamic): layer 0 whole in the oracle, every
  intermediate; the 64-layer stack under batch-permutation equivariance
  (per-tensor maxima do not depend on the order of the rows, everything else
  is row- or sequence-local, so reversing the batch reverses the output bit
  for bit).
* m130m_stack_static (batch 8, L 2048): the 24-layer stack calibrated on its
  64 sequences, then two properties on the evaluation batch (a sequence alone
  gives its row of the batch; a prefill continued by decode steps gives the
  longer prefill); the calibrated maxima of layer 0 cover the oracle's over
  one calibration sequence; layers 0, 11 and 23 as static layers whose
  parameters the oracle calibrates itself, run on the whole batch, one whole
  sequence recomputed by the oracle.
* m2p7b_decode (batch 16): layers 0 and 63 as one-layer graph-replayed decode
  stacks from an 8-token prefill that the oracle runs too, every step bit for
  bit; the 64-layer stack's graph replays equal its eager steps.
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
def test_m2p7b_layer0_full_size_whole(B):
    """Layer 0 of the 2.7B stack at 4 x 4096: the oracle recomputes all of it."""
    from quantized_state_space_fwht_amd.runtime import Mamba2Layer
    w = configs.get("m2p7b_stack")
    s = w.shape
    params = synth.workload_params(w, 0)
    u = synth.workload_activations(w)
    T = w.batch * w.seqlen
    out_o, r, cache_o, st_o = O.layer_prefill(O.prepare_layer(params), s, prenorm(u),
                                              scan=ssm_scan_pot_c)
    want = u + out_o
    layer = Mamba2Layer(s, params, prenorm_residual=True)
    h = layer.prefill(dev(u))  # as the stack runs it: no intermediates kept
    assert_same_float(host(h), want, "layer 0 output")
    check_caches_and_record(layer, cache_o, r, st_o)
    B.keep_intermediates(True)
    try:
        layer.reset_stats()
        h = layer.prefill(dev(u))
        check_intermediates(layer, r, T, s)
        assert_same_float(host(h), want, "layer 0 output (intermediates kept)")
    finally:
        B.keep_intermediates(False)


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
def test_m130m_static_stack_full_size(B):
    from quantized_state_space_fwht_amd.runtime import Mamba2Layer, Mamba2Stack
    w = configs.get("m130m_stack_static")
    s = w.shape
    params = [synth.workload_params(w, l) for l in range(w.nlayers)]
    stack = Mamba2Stack(s, params)
    calib = synth.calibration_sequences(w)
    stack.calibrate([dev(c) for c in calib])
    # the layer-0 maxima cover the oracle's over calibration sequence 0
    _, _, _, st0 = O.layer_prefill(O.prepare_layer(params[0]), s, prenorm(calib[0]),
                                   scan=ssm_scan_pot_c)
    qp0 = stack.layers[0].qparams()
    assert np.float32(qp0.stat_amax[0]) >= np.float32(st0.amax_u)
    assert np.float32(qp0.stat_amax[1]) >= np.float32(st0.amax_g)
    assert np.float32(qp0.stat_amax[2]) >= np.float32(st0.amax_xbc)
    assert all(int(a) >= int(b) for a, b in zip(qp0.stat_amax_q16, st0.amax_q16))
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
    # static layers with parameters the oracle calibrates, on the whole batch
    cal_short = [c[:, :256] for c in calib[:2]]
    for l in (0, 11, w.nlayers - 1):
        prep = O.prepare_layer(params[l])
        qps, _ = O.calibrate_stack([prep], s, cal_short)
        qp = qps[0]
        layer = Mamba2Layer(s, params[l], mode="static", prenorm_residual=True)
        layer.set_static(B.StaticParams(tuple(qp.scoe), tuple(qp.sshift), tuple(qp.p)))
        hl = host(layer.prefill(dev(u)))
        out_o, _, cache_o, _ = O.layer_prefill(prep, s, prenorm(u[bsel:bsel + 1]), "static", qp,
                                               scan=ssm_scan_pot_c)
        assert_same_float(hl[bsel:bsel + 1], u[bsel:bsel + 1] + out_o, f"layer {l} sequence")
        assert_exact(host(layer.cache_t["ssm_state"])[bsel], cache_o["ssm_state"][0],
                     f"layer {l} state")
        assert_exact(host(layer.cache_t["conv_state"])[bsel], cache_o["conv_state"][0],
                     f"layer {l} conv window")


# ----------------------------------------------------------------- m2p7b_decode
@pytest.mark.parametrize("layer_idx", [0, 63])
def test_m2p7b_decode_layer_full_size(B, layer_idx):
    """One 2.7B layer at batch 16, graph-replayed as the decode benchmark runs its
    layers, from an 8-token prefill that the oracle runs too."""
    from quantized_state_space_fwht_amd.runtime import DecodeGraph, Mamba2Stack
    w = configs.get("m2p7b_decode")
    s = w.shape
    L0, K = 8, 4
    wl = configs.with_len(w, w.batch, L0 + K)
    params = synth.workload_params(w, layer_idx)
    u = synth.workload_activations(wl)
    prep = O.prepare_layer(params)
    _, _, cache, _ = O.layer_prefill(prep, s, prenorm(u[:, :L0]))
    stack = Mamba2Stack(s, [params])
    stack.prefill(dev(u[:, :L0]))
    layer = stack.layers[0]
    assert_exact(host(layer.cache_t["ssm_state"]), cache["ssm_state"], "state after prefill")
    g = DecodeGraph(stack, w.batch)
    for t in range(L0, L0 + K):
        out_o, _, cache, _ = O.layer_decode(prep, s, prenorm(u[:, t]), cache)
        got = host(g.step(dev(u[:, t])))
        assert_same_float(got, u[:, t] + out_o, f"layer {layer_idx} step {t}")
        assert_exact(host(layer.cache_t["ssm_state"]), cache["ssm_state"], f"state step {t}")
        assert_exact(host(layer.cache_t["conv_state"]), cache["conv_state"], f"conv step {t}")


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
