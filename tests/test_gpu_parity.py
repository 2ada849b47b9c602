"""GPU parity: every C-ABI call against the CPU oracle on the same seeded inputs.

Integer / fixed-point results must match bit for bit; float outputs must stay
within 1e-3 max relative error (they are expected to be bit-identical too,
since both sides run the same IEEE float32 operations).  Inputs of each step
come from the oracle's own upstream values, so a mismatch names its step.
"""
import ctypes

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


def dev(a, dtype=None):
    t = torch.as_tensor(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda().contiguous()


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


def assert_float(got, want, what, tol=1e-3):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    denom = max(np.max(np.abs(want)), 1e-30)
    err = np.max(np.abs(got - want)) / denom if want.size else 0.0
    assert err <= tol, f"{what}: max relative error {err:.3e} > {tol}"


# --------------------------------------------------------------------------- a1 / a2
@pytest.mark.parametrize("rows,k", [(1, 256), (37, 768), (2048, 768), (5, 2560), (0, 512)])
@pytest.mark.parametrize("mode", ["dynamic", "static"])
def test_hadamard_quant(B, rows, k, mode):
    rng = np.random.default_rng(rows * 7 + k)
    x = (rng.standard_normal((rows, k)) * 2).astype(np.float32)
    if rows:
        x[:, [3, k // 2]] *= 50
    scoe, sshift = (23456, 17) if mode == "static" else (0, 0)
    q = torch.empty((rows, k), dtype=torch.int8, device="cuda")
    s = torch.empty(1, dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.float32, device="cuda")
    B.fm_hadamard_quant(dev(x), B.STATIC if mode == "static" else B.DYNAMIC, scoe, sshift, q, s, st)
    oq, os_, oamax, _ = O.hadamard_quant(x, mode, scoe if mode == "static" else None,
                                         sshift if mode == "static" else None)
    assert_exact(host(q), oq, "codes")
    assert host(s)[0] == os_, (host(s)[0], os_)
    assert host(st)[0] == oamax


# --------------------------------------------------------------------------- a3 / a9
@pytest.mark.parametrize("m,n,k", [(1, 1, 64), (17, 40, 64), (300, 1160, 256), (2048, 3352, 768),
                                   (2048, 768, 1536), (129, 257, 512),
                                   # tile shapes 64x64 / 64x128 / 128x128 and k-step counts
                                   # below, at and past the depth of the load ring
                                   (200, 300, 128), (130, 1100, 192), (2048, 1536, 256),
                                   (1000, 4100, 448), (70, 90, 320),
                                   # large products (256 x 128 tiles, direct-to-LDS stages):
                                   # 1 and 2 k-steps, a ragged edge with 5, and 40
                                   (4096, 8192, 64), (4096, 8192, 128), (4100, 8200, 320),
                                   (4096, 8192, 2560),
                                   # few-row path (m <= 64, k % 256 == 0): decode shapes, ragged n
                                   (16, 10576, 2560), (16, 2560, 5120), (1, 33, 256),
                                   (3, 1160, 256), (40, 300, 768), (64, 777, 1536)])
def test_w8a8_gemm(B, m, n, k):
    rng = np.random.default_rng(m + n + k)
    a = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    b = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    sa, sb = np.float32(0.0123), np.float32(0.00071)
    acc = torch.empty((m, n), dtype=torch.int32, device="cuda")
    out = torch.empty((m, n), dtype=torch.float32, device="cuda")
    B.fm_w8a8_gemm(dev(a), dev(b), dev(np.array([sa])), dev(np.array([sb])), acc, out)
    oacc, oout = O.w8a8_gemm(a, b, sa, sb)
    assert_exact(host(acc), oacc, "acc")
    assert_float(host(out), oout, "out")
    assert np.array_equal(host(out), oout)


# --------------------------------------------------------------------------- a6 (NAU)
@pytest.mark.parametrize("fn", ["exp", "softplus", "silu"])
def test_nau_elementwise(B, fn):
    """Every Q.16 input in [-2^23, 2^23] plus 2^20 random int32 values."""
    rng = np.random.default_rng(17)
    x = np.concatenate([np.arange(-(1 << 23), (1 << 23) + 1, dtype=np.int64),
                        rng.integers(-(1 << 31), (1 << 31), size=1 << 20),
                        np.array([-(1 << 31), (1 << 31) - 1, -1, 0, 1])]).astype(np.int32)
    code = {"exp": B.NAU_EXP, "softplus": B.NAU_SOFTPLUS, "silu": B.NAU_SILU}[fn]
    t_y = torch.empty(x.shape, dtype=torch.int32, device="cuda")
    B.fm_nau_eval(code, dev(x), t_y)
    xi = x.astype(np.int64)
    want = {"exp": lambda: O.exp_q16(np.minimum(xi, 0)), "softplus": lambda: O.softplus_q16(xi),
            "silu": lambda: O.silu_q16(xi)}[fn]()
    assert_exact(host(t_y), want, fn)


# --------------------------------------------------------------------------- a4 / a5
def _conv_case(shape, batch, length, seed):
    rng = np.random.default_rng(seed)
    ch = shape.conv_ch
    params = synth.layer_params(shape, 1000 + seed)
    w_q, p_w, b_q16 = O.conv_weight_prep(params["conv_w"], params["conv_b"])
    xbc = (rng.standard_normal((batch * length, ch)) * 2).astype(np.float32)
    return params, w_q, p_w, b_q16, xbc


@pytest.mark.parametrize("wname,batch,length", [("tiny_layer", 1, 256), ("tiny_layer", 3, 37),
                                                ("m130m_layer", 1, 2048), ("m130m_layer", 2, 5)])
@pytest.mark.parametrize("mode", ["dynamic", "static"])
@pytest.mark.parametrize("with_state", [False, True])
def test_conv1d_pot(B, wname, batch, length, mode, with_state):
    s = configs.get(wname).shape
    di, N, ch = s.d_inner, s.dstate, s.conv_ch
    params, w_q, p_w, b_q16, xbc = _conv_case(s, batch, length, 5)
    # the standalone call gets its own weight prep on the device
    t_wq = torch.empty((ch, 4), dtype=torch.int8, device="cuda")
    t_pw = torch.empty(ch, dtype=torch.int32, device="cuda")
    t_bq = torch.empty(ch, dtype=torch.int32, device="cuda")
    _device_conv_prep(B, s, params, t_wq, t_pw, t_bq)
    assert_exact(host(t_wq), w_q, "conv w_q")
    assert_exact(host(t_pw), p_w, "conv p_w")
    assert_exact(host(t_bq), b_q16, "conv b_q16")
    rng = np.random.default_rng(9)
    state = rng.integers(-127, 128, size=(batch, ch, 3)).astype(np.int8) if with_state else None
    p_fixed = (2, 7, 8, 6) if mode == "static" else None
    # oracle
    xbc_q, p_c, amax = O.xbc_pot_quant(xbc, None if p_fixed is None else p_fixed[0])
    a, _, st_out = O.conv1d_pot(xbc_q.reshape(batch, length, ch), w_q, p_w, b_q16, p_c, state)
    xq, bq, cq, ps, amaxes, _ = O.silu_requant(a, di, N, None if p_fixed is None else p_fixed[1:])
    # gpu: xbc handed over as a strided view inside a wider row (as in the layer)
    stride = ch + 24
    wide = np.zeros((batch * length, stride), np.float32)
    wide[:, 8:8 + ch] = xbc
    t_wide = dev(wide)
    T = batch * length
    out = {k: torch.empty(shp, dtype=torch.int8, device="cuda") for k, shp in
           (("xbc_q", (T, ch)), ("x", (T, di)), ("b", (T, N)), ("c", (T, N)))}
    t_st_out = torch.zeros((batch, ch, 3), dtype=torch.int8, device="cuda")
    t_p = torch.zeros(4, dtype=torch.int32, device="cuda")
    t_stats = torch.zeros(4, dtype=torch.int32, device="cuda")
    B.fm_conv1d_pot(t_wide[:, 8:], stride, batch, length, di, N, t_wq, t_pw, t_bq,
                    B.STATIC if mode == "static" else B.DYNAMIC,
                    None if p_fixed is None else dev(np.array(p_fixed, np.int32)),
                    None if state is None else dev(state), t_st_out, out["xbc_q"], out["x"],
                    out["b"], out["c"], t_p, t_stats)
    assert_exact(host(out["xbc_q"]), xbc_q, "xbc_q")
    assert_exact(host(t_p), (p_c,) + tuple(ps), "exponents")
    assert_exact(host(out["x"]), xq.reshape(T, di), "x codes")
    assert_exact(host(out["b"]), bq.reshape(T, N), "B codes")
    assert_exact(host(out["c"]), cq.reshape(T, N), "C codes")
    assert_exact(host(t_st_out), st_out, "conv state")
    stats = host(t_stats)
    assert stats[0] == np.float32(amax).view(np.int32)
    assert_exact(stats[1:], amaxes, "Q.16 maxima")


def test_conv1d_pot_wave_exponents_far_apart(B):
    """Dynamic conv whose 64-channel groups and 16-step runs differ by many
    octaves: silent groups (zero weights and bias: all-zero SiLU values), groups
    with a tiny bias and tiny inputs, ordinary ones and large ones, and a run of
    silent steps across every group.  Between its two passes the kernel holds
    each wave's values as 16-bit words at the wave's own power-of-two exponent;
    these inputs spread those exponents from the top of the exponent range (24,
    silent waves) to the tensor's own, so the words are formed by left and by
    right shifts and brought back onto the tensor's grid by rounding shifts from
    1 to past 16 places.  Ragged length, two sequences, a carried window: codes
    and exponents equal the oracle's."""
    s = configs.get("m130m_layer").shape
    di, N, ch = s.d_inner, s.dstate, s.conv_ch
    batch, length = 2, 83
    params, _, _, _, _ = _conv_case(s, batch, length, 7)
    groups = ch // 64
    kind = np.arange(groups) % 4            # 0 silent, 1 tiny, 2 ordinary, 3 large
    w = np.asarray(params["conv_w"], np.float32).copy()
    b = np.asarray(params["conv_b"], np.float32).copy()
    gsel = np.repeat(kind, 64)
    w[gsel == 0] = 0.0
    b[gsel == 0] = 0.0
    b[gsel == 1] = 2e-4
    b[gsel == 3] *= 500.0
    params = dict(params, conv_w=w, conv_b=b)
    w_q, p_w, b_q16 = O.conv_weight_prep(params["conv_w"], params["conv_b"])
    rng = np.random.default_rng(13)
    gain = np.array([0.0, 1e-5, 1.0, 400.0], np.float32)[gsel]
    xbc = (rng.standard_normal((batch * length, ch)) * gain[None, :]).astype(np.float32)
    xbc[16:48] = 0.0
    t_wq = torch.empty((ch, 4), dtype=torch.int8, device="cuda")
    t_pw = torch.empty(ch, dtype=torch.int32, device="cuda")
    t_bq = torch.empty(ch, dtype=torch.int32, device="cuda")
    _device_conv_prep(B, s, params, t_wq, t_pw, t_bq)
    assert_exact(host(t_bq), b_q16, "conv b_q16")
    state = np.zeros((batch, ch, 3), np.int8)
    state[:, gsel == 3] = 100
    xbc_q, p_c, amax = O.xbc_pot_quant(xbc, None)
    a, _, st_out = O.conv1d_pot(xbc_q.reshape(batch, length, ch), w_q, p_w, b_q16, p_c, state)
    xq, bq, cq, ps, amaxes, _ = O.silu_requant(a, di, N, None)
    T = batch * length
    out = {k: torch.empty(shp, dtype=torch.int8, device="cuda") for k, shp in
           (("xbc_q", (T, ch)), ("x", (T, di)), ("b", (T, N)), ("c", (T, N)))}
    t_st_out = torch.zeros((batch, ch, 3), dtype=torch.int8, device="cuda")
    t_p = torch.zeros(4, dtype=torch.int32, device="cuda")
    t_stats = torch.zeros(4, dtype=torch.int32, device="cuda")
    B.fm_conv1d_pot(dev(xbc), ch, batch, length, di, N, t_wq, t_pw, t_bq, B.DYNAMIC, None,
                    dev(state), t_st_out, out["xbc_q"], out["x"], out["b"], out["c"], t_p,
                    t_stats)
    assert_exact(host(t_p), (p_c,) + tuple(ps), "exponents")
    assert_exact(host(out["x"]), xq.reshape(T, di), "x codes")
    assert_exact(host(out["b"]), bq.reshape(T, N), "B codes")
    assert_exact(host(out["c"]), cq.reshape(T, N), "C codes")
    assert_exact(host(t_st_out), st_out, "conv state")
    assert_exact(host(t_stats)[1:], amaxes, "Q.16 maxima")
    # the case spans the intended range: the B part holds only silent and tiny
    # groups (a high tensor exponent), x and C large ones next to silent groups
    assert ps[1] >= 16 and ps[0] <= 0 and ps[2] <= 0
    assert np.abs(xq).max() > 60 and (xq == 0).mean() > 0.2


def _device_conv_prep(B, s, params, t_wq, t_pw, t_bq):
    desc = B.LayerDesc(s.d_model, s.d_inner, s.nheads, s.headdim, s.dstate, 4, 0, 0)
    # keep every input tensor referenced until the asynchronous kernels have run
    src = {k: dev(np.asarray(params[k], np.float32))
           for k in ("w_in", "w_out", "conv_w", "conv_b", "A", "D")}
    tmp = {k: torch.empty(n, dtype=dt, device="cuda") for k, n, dt in (
        ("wi", (s.d_in_proj, s.d_model), torch.int8), ("si", 1, torch.float32),
        ("wo", (s.d_model, s.d_inner), torch.int8), ("so", 1, torch.float32),
        ("aq", s.nheads, torch.int32), ("dq", s.nheads, torch.int32))}
    ws = B.workspace(B.lib.fm_prepare_layer_workspace_size(ctypes.byref(desc)))
    B._check(B.lib.fm_prepare_layer(
        ctypes.byref(desc), src["w_in"].data_ptr(), src["w_out"].data_ptr(),
        src["conv_w"].data_ptr(), src["conv_b"].data_ptr(), src["A"].data_ptr(),
        src["D"].data_ptr(), tmp["wi"].data_ptr(), tmp["si"].data_ptr(), tmp["wo"].data_ptr(),
        tmp["so"].data_ptr(), t_wq.data_ptr(), t_pw.data_ptr(), t_bq.data_ptr(),
        tmp["aq"].data_ptr(), tmp["dq"].data_ptr(), ws.data_ptr(), ws.numel(), B._stream(None)))
    torch.cuda.synchronize()
    return tmp


# --------------------------------------------------------------------------- a6 / a7
@pytest.mark.parametrize("wname,batch,length,heads", [("tiny_layer", 1, 256, None),
                                                      ("tiny_layer", 2, 19, None),
                                                      ("m130m_layer", 1, 2048, None),
                                                      ("m130m_layer", 3, 5, 2),
                                                      ("m130m_layer", 1, 16, 2),
                                                      ("m130m_layer", 2, 33, 3),
                                                      ("m130m_layer", 3, 1, 4),
                                                      ("tiny_layer", 2, 1, None),
                                                      ("m2p7b_stack", 1, 300, 4),
                                                      # grids past the CU count: 4-wave
                                                      # workgroups with one B/C buffer, and
                                                      # 8-wave ones with two (d_state 128, 64)
                                                      ("m130m_layer", 2, 37, None),
                                                      ("m130m_layer", 16, 40, None),
                                                      ("tiny_layer", 5, 20, None),
                                                      ("tiny_layer", 64, 20, None),
                                                      # one row per wave at up to two
                                                      # workgroups per CU, d_state 64
                                                      ("tiny_layer", 3, 45, None)])
@pytest.mark.parametrize("with_state", [False, True])
def test_ssm_scan_pot(B, wname, batch, length, heads, with_state):
    s = configs.get(wname).shape
    H = heads or s.nheads
    P, N = s.headdim, s.dstate
    rng = np.random.default_rng(length + H)
    x = rng.integers(-127, 128, size=(batch, length, H, P)).astype(np.int8)
    bm = rng.integers(-127, 128, size=(batch, length, N)).astype(np.int8)
    cm = rng.integers(-127, 128, size=(batch, length, N)).astype(np.int8)
    stride = H + 5
    dt_wide = (rng.standard_normal((batch * length, stride)) * 2).astype(np.float32)
    dt_raw = dt_wide[:, :H].reshape(batch, length, H)
    dt_bias = rng.uniform(-4, -2, H).astype(np.float32)
    A = (-np.exp(rng.uniform(0, 2, H))).astype(np.float32)
    a_q16 = O.f32_to_i32_sat(np.rint(A * np.float32(65536)))
    d_q16 = np.full(H, 65536, np.int64)
    p = np.array([0, 7, 6, 7], np.int32)
    state = rng.integers(-(1 << 20), 1 << 20, size=(batch, H, P, N)).astype(np.int32) \
        if with_state else None
    dt, dA = O.dt_dA(dt_raw, dt_bias, a_q16)
    y, st = O.ssm_scan_pot(x, bm, cm, dt, dA, d_q16, p[2], p[3], state)
    t_y = torch.empty((batch, length, H, P), dtype=torch.int32, device="cuda")
    t_st = torch.empty((batch, H, P, N), dtype=torch.int32, device="cuda")
    t_dt = torch.empty((batch, length, H), dtype=torch.int32, device="cuda")
    t_da = torch.empty((batch, length, H), dtype=torch.int32, device="cuda")
    B.fm_ssm_scan_pot(dev(x), dev(bm), dev(cm), dev(dt_wide), stride, dev(dt_bias),
                      dev(a_q16, torch.int32), dev(d_q16, torch.int32), dev(p), batch, length, H,
                      P, N, None if state is None else dev(state), t_st, t_y, t_dt, t_da)
    assert_exact(host(t_dt), dt, "dt")
    assert_exact(host(t_da), dA, "dA")
    assert_exact(host(t_y), y, "y")
    assert_exact(host(t_st), st, "state")


def test_ssm_scan_saturates_like_the_oracle(B):
    """Extreme inputs: the int32 clamp of the state and of y must agree."""
    batch, length, H, P, N = 1, 40, 2, 8, 64
    x = np.full((batch, length, H, P), 127, np.int8)
    x[..., 1] = -127
    bm = np.full((batch, length, N), 127, np.int8)
    cm = np.full((batch, length, N), -127, np.int8)
    dt_raw = np.full((batch * length, H), 20000.0, np.float32)   # dt near 2^31 / 2^16
    dt_bias = np.zeros(H, np.float32)
    a_q16 = np.array([0, -3], np.int64)                          # decay exactly 1 / almost 1
    d_q16 = np.array([1 << 30, -(1 << 30)], np.int64)
    p = np.array([0, 7, -20, -20], np.int32)
    dt, dA = O.dt_dA(dt_raw.reshape(batch, length, H), dt_bias, a_q16)
    y, st = O.ssm_scan_pot(x, bm, cm, dt, dA, d_q16, p[2], p[3])
    assert np.any(np.abs(st) == 2 ** 31 - 1) or np.any(st == -2 ** 31)
    t_y = torch.empty((batch, length, H, P), dtype=torch.int32, device="cuda")
    t_st = torch.empty((batch, H, P, N), dtype=torch.int32, device="cuda")
    t_dt = torch.empty((batch, length, H), dtype=torch.int32, device="cuda")
    t_da = torch.empty((batch, length, H), dtype=torch.int32, device="cuda")
    B.fm_ssm_scan_pot(dev(x), dev(bm), dev(cm), dev(dt_raw), H, dev(dt_bias),
                      dev(a_q16, torch.int32), dev(d_q16, torch.int32), dev(p), batch, length, H,
                      P, N, None, t_st, t_y, t_dt, t_da)
    assert_exact(host(t_dt), dt, "dt (saturating)")
    assert_exact(host(t_y), y, "y (saturating)")
    assert_exact(host(t_st), st, "state (saturating)")


@pytest.mark.parametrize("batch", [1, 80, 160])
def test_ssm_scan_mixed_saturation(B, batch):
    """Some states reach the int32 clamp part-way through a long sequence (decay
    exactly 1, B and x of one sign) while others stay small: chunks before and
    after the crossing, and workgroups that never get near it, must all agree.
    Batches 1, 80 and 160 take the one-row, the 4-wave and the 8-wave layouts."""
    length, H, P, N = 181, 2, 16, 128
    rng = np.random.default_rng(11)
    x = rng.integers(-127, 128, size=(batch, length, H, P)).astype(np.int8)
    x[:, :, 1, :8] = 127                        # head 1, first 8 p: one sign
    bm = rng.integers(-127, 128, size=(batch, length, N)).astype(np.int8)
    bm[:, :, :64] = 127                         # n < 64: one sign
    cm = rng.integers(-127, 128, size=(batch, length, N)).astype(np.int8)
    dt_raw = np.empty((batch * length, H), np.float32)
    dt_raw[:, 0] = rng.uniform(-3, 0, batch * length)
    dt_raw[:, 1] = rng.uniform(8.5, 9.5, batch * length)   # dt near 9 in Q.16
    dt_bias = np.zeros(H, np.float32)
    a_q16 = np.array([-3 * 65536, 0], np.int64)            # head 1: decay exactly 1
    d_q16 = np.array([65536, 3 << 16], np.int64)
    p = np.array([0, 7, 0, 0], np.int32)
    state = rng.integers(-(1 << 20), 1 << 20, size=(batch, H, P, N)).astype(np.int32)
    state[0, 0, 8:] = 2 ** 31 - 5                          # one workgroup starts at the edge
    dt, dA = O.dt_dA(dt_raw.reshape(batch, length, H), dt_bias, a_q16)
    y, st = O.ssm_scan_pot(x, bm, cm, dt, dA, d_q16, p[2], p[3], state)
    assert np.any(st[0, 1, :8, :64] == 2 ** 31 - 1)
    assert np.all(np.abs(st[0, 1, 8:]) < 2 ** 31 - 1)
    t_y = torch.empty((batch, length, H, P), dtype=torch.int32, device="cuda")
    t_st = torch.empty((batch, H, P, N), dtype=torch.int32, device="cuda")
    t_dt = torch.empty((batch, length, H), dtype=torch.int32, device="cuda")
    t_da = torch.empty((batch, length, H), dtype=torch.int32, device="cuda")
    B.fm_ssm_scan_pot(dev(x), dev(bm), dev(cm), dev(dt_raw), H, dev(dt_bias),
                      dev(a_q16, torch.int32), dev(d_q16, torch.int32), dev(p), batch, length, H,
                      P, N, dev(state), t_st, t_y, t_dt, t_da)
    assert_exact(host(t_y), y, "y (mixed)")
    assert_exact(host(t_st), st, "state (mixed)")


# --------------------------------------------------------------------------- a8
@pytest.mark.parametrize("wname,rows", [("tiny_layer", 256), ("m130m_layer", 2048),
                                        ("m2p7b_stack", 33)])
@pytest.mark.parametrize("mode", ["dynamic", "static"])
def test_gate_norm_quant(B, wname, rows, mode):
    s = configs.get(wname).shape
    di = s.d_inner
    rng = np.random.default_rng(rows)
    y = rng.integers(-(1 << 22), 1 << 22, size=(rows, di)).astype(np.int32)
    zw = (rng.standard_normal((rows, di + 64)) * 3).astype(np.float32)
    z = zw[:, 32:32 + di]
    w = (1 + 0.1 * rng.standard_normal(di)).astype(np.float32)
    p = np.array([0, 9, 0, 0], np.int32)
    scoe, sshift = (20000, 9) if mode == "static" else (0, 0)
    oq, os_, oamax, on = O.gate_norm_quant(y, z, p[1] + 8, w, mode,
                                           scoe if mode == "static" else None,
                                           sshift if mode == "static" else None)
    t_zw = dev(zw)
    q = torch.empty((rows, di), dtype=torch.int8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.float32, device="cuda")
    normed = torch.empty((rows, di), dtype=torch.float32, device="cuda")
    B.fm_gate_norm_quant(dev(y), t_zw[:, 32:], di + 64, dev(p), dev(w), rows, di,
                         B.STATIC if mode == "static" else B.DYNAMIC, scoe, sshift, q, sc, st,
                         normed)
    assert np.array_equal(host(normed), on), "normed values differ"
    assert_exact(host(q), oq, "g codes")
    assert host(sc)[0] == os_
    assert host(st)[0] == oamax


# --------------------------------------------------------------------------- layer
def _layer_case(wname, batch=None, seqlen=None, mode="dynamic"):
    w = configs.with_len(configs.get(wname), batch, seqlen)
    params = synth.workload_params(w, 0)
    u = synth.workload_activations(w)
    return w, params, u


def _check_layer_intermediates(layer, r, T, s):
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


@pytest.mark.parametrize("wname,batch,seqlen", [("tiny_layer", None, None), ("tiny_layer", 3, 50),
                                                ("tiny_layer", 1, 1), ("tiny_layer", 4, 1),
                                                ("m130m_layer", None, None)])
def test_layer_prefill_dynamic(B, wname, batch, seqlen):
    from quantized_state_space_fwht_amd.runtime import Mamba2Layer
    w, params, u = _layer_case(wname, batch, seqlen)
    s = w.shape
    prep = O.prepare_layer(params)
    out_o, r, cache_o, st_o = O.layer_prefill(prep, s, u)
    layer = Mamba2Layer(s, params)
    assert_exact(host(layer.t["w_in_q"]), prep["w_in_q"], "W_in codes")
    assert host(layer.t["s_w_in"])[0] == prep["s_w_in"]
    assert_exact(host(layer.t["w_out_q"]), prep["w_out_q"], "W_out codes")
    assert_exact(host(layer.t["a_q16"]), prep["A_q16"], "A_q16")
    out = layer.prefill(dev(u), opts=B.layer_opts(keep=True))
    torch.cuda.synchronize()
    T = w.batch * w.seqlen
    _check_layer_intermediates(layer, r, T, s)
    assert np.array_equal(host(out), out_o), "layer output"
    assert_exact(host(layer.cache_t["ssm_state"]), cache_o["ssm_state"], "ssm state")
    assert_exact(host(layer.cache_t["conv_state"]), cache_o["conv_state"], "conv state")
    assert_exact(host(layer.cache_t["p"]), cache_o["p"], "cached exponents")
    qp = layer.qparams()
    assert qp.scale[0] == r["s_u"] and qp.scale[1] == r["s_g"]
    assert tuple(qp.p) == tuple(r["p"])
    assert qp.stat_amax[0] == np.float32(st_o.amax_u)
    assert qp.stat_amax[2] == np.float32(st_o.amax_xbc)
    assert list(qp.stat_amax_q16) == list(st_o.amax_q16)


# 64 rows: the largest one-token step of the fused five-kernel form; 65: the
# general launch sequence with the windows and states carried in
@pytest.mark.parametrize("batch", [2, 64, 65])
def test_layer_decode_continues_prefill(B, batch):
    from quantized_state_space_fwht_amd.runtime import Mamba2Layer
    w, params, u = _layer_case("tiny_layer", batch, 40)
    s = w.shape
    prep = O.prepare_layer(params)
    L0 = 30
    _, _, cache, _ = O.layer_prefill(prep, s, u[:, :L0])
    layer = Mamba2Layer(s, params)
    layer.prefill(dev(u[:, :L0]))
    for t in range(L0, 40):
        o_out, _, cache, _ = O.layer_decode(prep, s, u[:, t], cache)
        g_out = layer.decode(dev(u[:, t]))
        assert np.array_equal(host(g_out), o_out), f"decode step {t}"
        assert_exact(host(layer.cache_t["ssm_state"]), cache["ssm_state"], f"state step {t}")
        assert_exact(host(layer.cache_t["conv_state"]), cache["conv_state"], f"conv step {t}")


def test_static_stack_calibration_and_prefill(B):
    from quantized_state_space_fwht_amd.runtime import Mamba2Stack
    w = configs.with_len(configs.get("m130m_stack_static"), batch=2, seqlen=48)
    s = w.shape
    nl = 3
    params = [synth.workload_params(w, l) for l in range(nl)]
    calib = [synth.workload_activations(w, seed=sd) for sd in (100, 101)]
    u = synth.workload_activations(w, seed=200)
    preps = [O.prepare_layer(p) for p in params]
    qps, _ = O.calibrate_stack(preps, s, calib)
    h_o, caches_o, _ = O.stack_prefill(preps, s, u, "static", qps)
    stack = Mamba2Stack(s, params)
    stack.calibrate([dev(c) for c in calib])
    for layer, qp in zip(stack.layers, qps):
        sp = layer.static
        assert tuple(sp.scoe) == tuple(qp.scoe) and tuple(sp.sshift) == tuple(qp.sshift)
        assert tuple(sp.p) == tuple(qp.p)
    h = stack.prefill(dev(u))
    assert np.array_equal(host(h), h_o), "static stack output"
    for layer, c in zip(stack.layers, caches_o):
        assert_exact(host(layer.cache_t["ssm_state"]), c["ssm_state"], "stack state")
    # prefill then decode equals one longer prefill (static mode), on the GPU alone
    L0 = 40
    stack.prefill(dev(u[:, :L0]))
    outs = [host(stack.decode(dev(u[:, t]))) for t in range(L0, 48)]
    assert np.array_equal(np.stack(outs, axis=1), h_o[:, L0:]), "continuation"


@pytest.mark.parametrize("batch,seqlen", [(1, 37), (1, 2201)])
def test_dynamic_stack_prenorm_rows(B, batch, seqlen):
    """Dynamic-mode stack whose pre-norm passes see an odd row count (the last
    row pair half empty) and, at 2201 rows, more row pairs than resident
    workgroups (each workgroup loops over pairs): bit-exact against the oracle."""
    from quantized_state_space_fwht_amd.runtime import Mamba2Stack
    w = configs.with_len(configs.get("tiny_layer"), batch=batch, seqlen=seqlen)
    s = w.shape
    params = [synth.workload_params(w, l) for l in range(2)]
    u = synth.workload_activations(w, seed=300)
    preps = [O.prepare_layer(p) for p in params]
    h_o, caches_o, _ = O.stack_prefill(preps, s, u, "dynamic")
    stack = Mamba2Stack(s, params)
    h = stack.prefill(dev(u))
    assert np.array_equal(host(h), h_o), "dynamic stack output"
    for layer, c in zip(stack.layers, caches_o):
        assert_exact(host(layer.cache_t["ssm_state"]), c["ssm_state"], "stack state")


@pytest.mark.parametrize("fit", ["lsq", "minimax"])
@pytest.mark.parametrize("fn", ["exp", "softplus", "silu"])
def test_nau_other_knot_tables(B, fn, fit):
    """The unit with the fitted knot tables (alternative coefficients of the
    same form): every Q.16 input in [-2^22, 2^22] plus random int32 values,
    against the oracle evaluated with the same table."""
    knots = synth.nau_knot_tables()[fit]
    rng = np.random.default_rng(19)
    x = np.concatenate([np.arange(-(1 << 22), (1 << 22) + 1, dtype=np.int64),
                        rng.integers(-(1 << 31), (1 << 31), size=1 << 18),
                        np.array([-(1 << 31), (1 << 31) - 1, -1, 0, 1])]).astype(np.int32)
    code = {"exp": B.NAU_EXP, "softplus": B.NAU_SOFTPLUS, "silu": B.NAU_SILU}[fn]
    t_y = torch.empty(x.shape, dtype=torch.int32, device="cuda")
    B.fm_nau_eval_knots(code, knots, dev(x), t_y)
    xi = x.astype(np.int64)
    want = {"exp": lambda: O.exp_q16(np.minimum(xi, 0), knots),
            "softplus": lambda: O.softplus_q16(xi, knots),
            "silu": lambda: O.silu_q16(xi, knots)}[fn]()
    assert_exact(host(t_y), want, f"{fn} {fit}")


def test_ssm_scan_positive_a_is_decay_one(B):
    """A > 0 lies outside the method (A = -exp(.)): the exponential takes a
    positive argument as 0, so a positive a_q16 gives decay 2^16 and the same
    results as a_q16 = 0 (the oracle's reading of the unit on its domain)."""
    batch, length, H, P, N = 2, 70, 3, 8, 64
    rng = np.random.default_rng(77)
    x = rng.integers(-127, 128, size=(batch, length, H, P)).astype(np.int8)
    bm = rng.integers(-127, 128, size=(batch, length, N)).astype(np.int8)
    cm = rng.integers(-127, 128, size=(batch, length, N)).astype(np.int8)
    dt_raw = (rng.standard_normal((batch * length, H)) - 3).astype(np.float32)
    dt_bias = np.zeros(H, np.float32)
    d_q16 = np.full(H, 65536, np.int64)
    p = np.array([0, 0, 8, 8], np.int32)
    dt, dA = O.dt_dA(dt_raw.reshape(batch, length, H), dt_bias, np.zeros(H, np.int64))
    assert np.all(dA == 65536)
    y, st = O.ssm_scan_pot(x, bm, cm, dt, dA, d_q16, p[2], p[3])
    for a_pos in ([1, 65536, 1 << 30], [0, 0, 0]):
        t_y = torch.empty((batch, length, H, P), dtype=torch.int32, device="cuda")
        t_st = torch.empty((batch, H, P, N), dtype=torch.int32, device="cuda")
        t_dt = torch.empty((batch, length, H), dtype=torch.int32, device="cuda")
        t_da = torch.empty((batch, length, H), dtype=torch.int32, device="cuda")
        B.fm_ssm_scan_pot(dev(x), dev(bm), dev(cm), dev(dt_raw), H, dev(dt_bias),
                          dev(np.array(a_pos), torch.int32), dev(d_q16, torch.int32), dev(p),
                          batch, length, H, P, N, None, t_st, t_y, t_dt, t_da)
        assert_exact(host(t_da), dA, f"dA, a_q16 {a_pos}")
        assert_exact(host(t_y), y, f"y, a_q16 {a_pos}")
        assert_exact(host(t_st), st, f"state, a_q16 {a_pos}")
