"""GPU parity at the full sizes of the stack and decode workloads, on samples.

The whole stack runs on the GPU at its real shape and launch configuration;
for a few sampled layers (and decode steps) the oracle recomputes, from that
layer's actual input, every stage on outputs it can afford one by one:

* the Hadamard quantization of the layer input (whole tensor), dt / dA (whole
  tensor), the xBC exponent and codes (whole tensor);
* the in_proj GEMM and the out_proj GEMM + residual on sampled rows;
* the conv + SiLU + requantization on sampled channels over every step;
* the scan on sampled (batch, head, p) chains over every step, with the
  final states;
* gate + RMSNorm + rotation + quantization on sampled rows, under the
  tensor maximum the GPU used (itself bounded below by the sampled rows).

Static-mode layers are row- and sequence-local, so there the oracle
recomputes one whole sequence of the batch through the sampled layers.
Decode steps are small enough for the oracle to recompute whole layer steps
from the GPU's caches.
"""
import numpy as np
import pytest

import oracle as O
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


def sample_rows(T, rng, n=10):
    return np.unique(np.concatenate([[0, 1, T // 2, T - 2, T - 1], rng.integers(0, T, n)]))


def check_dynamic_layer(layer, prep, s, h_in, h_out, batch, L, rng):
    """Sampled stage-by-stage check of one pre-norm residual layer (dynamic mode)."""
    T, dm, di, N, H, P = batch * L, s.d_model, s.d_inner, s.dstate, s.nheads, s.headdim
    ch, dip = s.conv_ch, s.d_in_proj
    qp = layer.qparams()
    h2 = h_in.reshape(T, dm)
    # a10 + a1: pre-norm, rotation, per-tensor quantization (whole tensor)
    xin = O.rmsnorm_fixed_order(h2, np.ones(dm, np.float32))
    u_q, s_u, amax_u, _ = O.hadamard_quant(xin, "dynamic")
    assert_exact(layer.tap("u_q", torch.int8, (T, dm)).cpu().numpy(), u_q, "u_q")
    assert np.float32(qp.scale[0]) == s_u and np.float32(qp.stat_amax[0]) == amax_u
    # a3: in_proj on sampled rows
    v = layer.tap("v", torch.float32, (T, dip)).cpu().numpy()
    R = sample_rows(T, rng)
    _, v_R = O.w8a8_gemm(u_q[R], prep["w_in_q"], s_u, prep["s_w_in"])
    assert_same_float(v[R], v_R, "in_proj rows")
    # a4: xBC exponent and codes (whole tensor, from the GPU's in_proj output)
    xbc_q, p_c, _ = O.xbc_pot_quant(v[:, di:di + ch])
    assert qp.p[0] == p_c, ("p_c", qp.p[0], p_c)
    # a5: conv + SiLU + requant on sampled channels, every step
    p_x, p_B, p_C = qp.p[1], qp.p[2], qp.p[3]
    cx = np.sort(rng.choice(di, 8, replace=False))
    cb = np.sort(rng.choice(N, 4, replace=False))
    cc = np.sort(rng.choice(N, 4, replace=False))
    chans = np.concatenate([cx, di + cb, di + N + cc])
    a, _, _ = O.conv1d_pot(xbc_q.reshape(batch, L, ch)[:, :, chans], prep["conv_w_q"][chans],
                           prep["p_w"][chans], prep["conv_b_q16"][chans], p_c)
    x_s, b_s, c_s, _, amaxes, _ = O.silu_requant(a, len(cx), len(cb), (p_x, p_B, p_C))
    x_q = layer.tap("x_q", torch.int8, (T, di)).cpu().numpy()
    b_q = layer.tap("b_q", torch.int8, (T, N)).cpu().numpy()
    c_q = layer.tap("c_q", torch.int8, (T, N)).cpu().numpy()
    assert_exact(x_q[:, cx], x_s.reshape(T, -1), "x codes (sampled channels)")
    assert_exact(b_q[:, cb], b_s.reshape(T, -1), "B codes (sampled channels)")
    assert_exact(c_q[:, cc], c_s.reshape(T, -1), "C codes (sampled channels)")
    # the tensor exponents cover at least the sampled channels' maxima
    for m, p in zip(amaxes, (p_x, p_B, p_C)):
        assert O.pot_q16(m) >= p
    # a6: dt and dA (whole tensor)
    dt, dA = O.dt_dA(v[:, di + ch:].reshape(batch, L, H), prep["dt_bias"], prep["A_q16"])
    assert_exact(layer.tap("dt", torch.int32, (batch, L, H)).cpu().numpy(), dt, "dt")
    assert_exact(layer.tap("da", torch.int32, (batch, L, H)).cpu().numpy(), dA, "dA")
    # a7: sampled chains over every step, and their final states
    y = layer.tap("y", torch.int32, (batch, L, H, P)).cpu().numpy()
    state = host(layer.cache_t["ssm_state"])
    x4 = x_q.reshape(batch, L, H, P)
    b3, c3 = b_q.reshape(batch, L, N), c_q.reshape(batch, L, N)
    for _ in range(4):
        bb, hh, pp = int(rng.integers(batch)), int(rng.integers(H)), int(rng.integers(P))
        y_o, st_o = O.ssm_scan_pot(x4[bb:bb + 1, :, hh:hh + 1, pp:pp + 1], b3[bb:bb + 1],
                                   c3[bb:bb + 1], dt[bb:bb + 1, :, hh:hh + 1],
                                   dA[bb:bb + 1, :, hh:hh + 1], prep["D_q16"][hh:hh + 1],
                                   p_B, p_C)
        assert_exact(y[bb, :, hh, pp], y_o[0, :, 0, 0], f"y chain {(bb, hh, pp)}")
        assert_exact(state[bb, hh, pp], st_o[0, 0, 0], f"state chain {(bb, hh, pp)}")
    # a8: gate, RMSNorm, rotation, quantization on sampled rows
    y2 = y.reshape(T, di)
    g = O.gate(y2[R], v[R, :di], p_x + 8)
    normed = O.rmsnorm_fixed_order(g, prep["norm_w"])
    r = O.fwht256_f32(normed)
    amax_g = np.float32(qp.stat_amax[1])
    assert amax_g >= np.max(np.abs(r))
    g_q_R, s_g = O.quantize_codes(r, O.hadamard_scale(amax_g, "dynamic"))
    g_q = layer.tap("g_q", torch.int8, (T, di)).cpu().numpy()
    assert_exact(g_q[R], g_q_R, "g_q rows")
    assert np.float32(qp.scale[1]) == s_g
    # a9 + a10: out_proj and the residual on sampled rows
    _, out_R = O.w8a8_gemm(g_q[R], prep["w_out_q"], s_g, prep["s_w_out"])
    assert_same_float(h_out.reshape(T, dm)[R], h2[R] + out_R, "layer output rows")
    assert tuple(host(layer.cache_t["p"])) == (p_c, p_x, p_B, p_C)


def test_m2p7b_stack_full_size_sampled(B):
    """64 layers, 2.7B shapes, batch 4, L 4096, dynamic scales; layers 0 and 63 checked."""
    from quantized_state_space_fwht_amd.runtime import Mamba2Stack
    w = configs.get("m2p7b_stack")
    s = w.shape
    check = {0, w.nlayers - 1}
    stack = Mamba2Stack(s, (synth.workload_params(w, l) for l in range(w.nlayers)))
    h = dev(synth.workload_activations(w))
    rng = np.random.default_rng(3)
    B.keep_intermediates(True)
    try:
        for l, layer in enumerate(stack.layers):
            layer.reset_stats()
            h_next = layer.prefill(h)
            if l in check:
                prep = O.prepare_layer(synth.workload_params(w, l))
                check_dynamic_layer(layer, prep, s, host(h), host(h_next), w.batch, w.seqlen,
                                    rng)
            h = h_next
    finally:
        B.keep_intermediates(False)
    assert np.all(np.isfinite(host(h)))


def test_m130m_static_stack_full_size_sampled(B):
    """24 layers, 130M shapes: calibration on 64 sequences, then batch 8 x L 2048 static.

    The static parameters must be the oracle's conversion of the GPU's
    calibration maxima; sampled layers are recomputed by the oracle for one
    whole sequence of the evaluation batch (static mode is sequence-local).
    """
    from quantized_state_space_fwht_amd.runtime import Mamba2Stack
    w = configs.get("m130m_stack_static")
    s = w.shape
    params = [synth.workload_params(w, l) for l in range(w.nlayers)]
    stack = Mamba2Stack(s, params)
    stack.calibrate([dev(c) for c in synth.calibration_sequences(w)])
    for layer in stack.layers:
        qp = layer.qparams()
        st = O.Stats()
        st.amax_u, st.amax_g, st.amax_xbc = (float(np.float32(qp.stat_amax[0])),
                                             float(np.float32(qp.stat_amax[1])),
                                             float(np.float32(qp.stat_amax[2])))
        st.amax_q16 = [int(m) for m in qp.stat_amax_q16]
        want = O.qparams_from_stats(st)
        sp = layer.static
        assert tuple(sp.scoe) == tuple(want.scoe) and tuple(sp.sshift) == tuple(want.sshift)
        assert tuple(sp.p) == tuple(want.p)
    # the accumulated maxima cover a calibration sequence recomputed by the oracle (layer 0)
    c0 = synth.calibration_sequences(w)[0]
    xin0 = O.rmsnorm_fixed_order(c0.reshape(-1, s.d_model), np.ones(s.d_model, np.float32))
    _, _, _, st0 = O.layer_prefill(O.prepare_layer(params[0]), s,
                                   xin0.reshape(1, w.seqlen, s.d_model))
    qp0 = stack.layers[0].qparams()
    assert np.float32(qp0.stat_amax[0]) >= np.float32(st0.amax_u)
    assert np.float32(qp0.stat_amax[2]) >= np.float32(st0.amax_xbc)
    assert all(int(a) >= int(b) for a, b in zip(qp0.stat_amax_q16, st0.amax_q16))

    u = synth.eval_batch(w)
    check = {0, 11, w.nlayers - 1}
    bsel = 5
    h = dev(u)
    for l, layer in enumerate(stack.layers):
        h_next = layer.prefill(h)
        if l in check:
            prep = O.prepare_layer(params[l])
            h_b = host(h)[bsel]
            xin = O.rmsnorm_fixed_order(h_b, np.ones(s.d_model, np.float32))
            sp = layer.static
            qpo = O.QParams(scoe=tuple(sp.scoe), sshift=tuple(sp.sshift), p=tuple(sp.p))
            out_o, _, cache_o, _ = O.layer_prefill(prep, s, xin[None], "static", qpo)
            assert_same_float(host(h_next)[bsel], h_b + out_o[0], f"layer {l} sequence {bsel}")
            assert_exact(host(layer.cache_t["ssm_state"])[bsel], cache_o["ssm_state"][0],
                         f"layer {l} state")
            assert_exact(host(layer.cache_t["conv_state"])[bsel], cache_o["conv_state"][0],
                         f"layer {l} conv window")
        h = h_next


def test_m2p7b_decode_full_size_sampled(B):
    """64 layers, 2.7B shapes, batch 16: 1024-token seeding prefill, then decode steps.

    For sampled (step, layer) pairs the oracle recomputes the whole layer step
    from the GPU's input and the GPU's caches before the step.
    """
    from quantized_state_space_fwht_amd.runtime import Mamba2Stack
    w = configs.get("m2p7b_decode")
    s = w.shape
    stack = Mamba2Stack(s, (synth.workload_params(w, l) for l in range(w.nlayers)))
    stack.prefill(dev(synth.workload_activations(w)))
    check_layers = {0, w.nlayers - 1}
    check_steps = {0, 1, 37}
    preps = {l: O.prepare_layer(synth.workload_params(w, l)) for l in check_layers}
    steps = max(check_steps) + 1
    for t in range(steps):
        h = dev(synth.decode_step_input(w, t))
        for l, layer in enumerate(stack.layers):
            probe = t in check_steps and l in check_layers
            if probe:
                cache = {k: host(v).copy() for k, v in layer.cache_t.items()}
                h_in = host(h)
            h = layer.decode(h)
            if probe:
                xin = O.rmsnorm_fixed_order(h_in, np.ones(s.d_model, np.float32))
                cache_o = {"conv_state": cache["conv_state"], "ssm_state": cache["ssm_state"],
                           "p": cache["p"].astype(np.int64)}
                out_o, _, new_o, _ = O.layer_decode(preps[l], s, xin, cache_o)
                assert_same_float(host(h), h_in + out_o, f"step {t} layer {l} output")
                assert_exact(host(layer.cache_t["ssm_state"]), new_o["ssm_state"],
                             f"step {t} layer {l} state")
                assert_exact(host(layer.cache_t["conv_state"]), new_o["conv_state"],
                             f"step {t} layer {l} conv window")
    assert np.all(np.isfinite(host(h)))
