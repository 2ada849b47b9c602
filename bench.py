#!/usr/bin/env python3
"""Benchmark: quantized Mamba2 mixer prefill tokens/s on one MI355X.

One step = one full prefill pass of the workload over one batch of seeded
synthetic input already resident in HBM: per layer the pre-norm (stacks),
Hadamard-quant, in_proj W8A8 GEMM, PoT conv1d + SiLU, NAU dt / decay +
fixed-point scan, gate + RMSNorm + Hadamard-quant, out_proj W8A8 GEMM and the
residual add.  Default workload: the 64-layer Mamba2-2.7B-shaped stack, batch
4, L 4096, dynamic scales (the largest prefill configuration that fits one
GPU).

Prints ONE JSON line.  `roofline` describes the dominant kernel (the scan),
timed live with HIP events the library records around that kernel on the
layer's stream inside the timed region; `stages` times every stage of a layer
the same way in one extra pass and gives each its own roofline fraction.  The
other workloads (one 130M layer, the 24-layer static 130M stack, the 2.7B
decode) are extra keys.  `cpu_baseline` times the CPU oracle (test
infrastructure, never tuned) on a bounded sample of the headline workload on
the host cores.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Mamba2 layer prefill tokens/s (W8A8+PoT SSM); % of i8 MFMA / HBM peak"
# MI355X: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz = 39.32e12 vector lane-operations/s
# (float64 FMA runs at this rate: 78.6 TFLOP/s counting an FMA as 2).
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
# algorithmic integer work per state element (b, head, p, n) per time step of
# the scan: 3 multiplies (dA*h, (dt*x)*B, C*h), 3 additions (the two rounded
# terms, the y accumulation) and 2 rounding shifts
SCAN_OPS_PER_ELEMENT_STEP = 8
COPY_PROBE_BYTES = 256 << 20
HBM_PEAK_GBS = 8000.0
I8_MFMA_PEAK_TOPS = 5000.0   # MI355X dense int8 matrix rate, 5.0 POP/s
HEADLINE_WORKLOAD = "m2p7b_stack"
DECODE_WORKLOAD = "m2p7b_decode"
STUDY_WORKLOAD = "m130m_stack_static"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def scan_source_hash():
    """Hash of the sources the scan kernel is compiled from (its file and the
    device headers it inlines): counters taken on another build are stale."""
    h = hashlib.sha256()
    for rel in (("quantized_state_space_fwht_amd", "csrc", "fm_scan.hip"),
                ("quantized_state_space_fwht_amd", "csrc", "fm_device.hpp"),
                ("quantized_state_space_fwht_amd", "csrc", "fm_internal.hpp"),
                ("include", "fm.h")):
        with open(os.path.join(ROOT, *rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload, per_launch_units):
    """HBM bytes per scan launch from committed rocprofv3 counter runs, if still current."""
    p = os.path.join(ROOT, "profiles", f"scan_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("scan_source_sha256_16") != scan_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def host_cpu():
    """What the host offers: logical CPUs, the ones this process may run on, the
    model string, and the BLAS thread count numpy's products use."""
    try:
        usable = len(os.sched_getaffinity(0))
    except Exception:
        usable = os.cpu_count()
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas = None
    return {"nproc": os.cpu_count(), "usable": usable, "model": model, "blas_threads": blas}


def cpu_baseline(w, sample_layers=2, sample_batch=1, sample_len=4096):
    """The oracle as it stands (numpy) on a bounded sample of the workload.

    Stacks: the first `sample_layers` layers over `sample_batch` x `sample_len`
    tokens of the same seeded input (about 10-20 s of CPU work); every layer of a
    stack costs the same and the oracle's cost is linear in tokens, so the
    whole stack's rate is the sample's tokens / (its time x layers / sample
    layers), reported beside the measured sample.  A single layer runs whole
    prefill passes until at least 10 s of work."""
    import oracle as O
    from quantized_state_space_fwht_amd import configs, synth
    cpu = host_cpu()
    if w.nlayers == 1:
        prep = O.prepare_layer(synth.workload_params(w, 0))
        u = synth.workload_activations(w)
        reps, t0 = 0, time.perf_counter()
        while reps < 30:
            O.layer_prefill(prep, w.shape, u)
            reps += 1
            if time.perf_counter() - t0 >= 10.0:
                break
        dt = time.perf_counter() - t0
        value = w.tokens * reps / dt
        sample = (f"{reps} full oracle prefill pass(es) of the workload ({w.batch}x{w.seqlen} "
                  f"tokens, seeds as the GPU run), {dt:.1f} s")
        measured = {"seconds": round(dt, 2), "tokens": w.tokens * reps, "layers": 1}
    else:
        nl = min(sample_layers, w.nlayers)
        preps = [O.prepare_layer(synth.workload_params(w, l)) for l in range(nl)]
        u = synth.workload_activations(configs.with_len(w, batch=sample_batch, seqlen=sample_len))
        qps = None
        if w.mode == "static":
            qps, _ = O.calibrate_stack(preps, w.shape, [u])
        t0 = time.perf_counter()
        O.stack_prefill(preps, w.shape, u, w.mode, qps)
        dt = time.perf_counter() - t0
        tokens = sample_batch * sample_len
        value = tokens / (dt * w.nlayers / nl)
        sample = (f"the first {nl} of {w.nlayers} layers over {sample_batch}x{sample_len} "
                  f"tokens of the same seeded input, {dt:.1f} s; extrapolated linearly to all "
                  f"{w.nlayers} layers (identical cost per layer, linear in tokens)")
        measured = {"seconds": round(dt, 2), "tokens": tokens, "layers": nl,
                    "tokens_per_s_of_the_sample_layers": round(tokens / dt, 1)}
    return {"value": round(value, 1), "unit": "tokens/s", "cores": cpu["usable"],
            "kind": "oracle", "sample": sample + "; numpy: the matrix products on "
            f"{cpu['blas_threads']} BLAS threads, elementwise work on one",
            "measured": measured, "host": cpu}


FP64_PEAK_TFLOPS = 78.6   # MI355X float64 vector / matrix rate


def measured_copy_gbs(torch, nbytes=512 << 20, reps=10):
    """Achievable HBM bandwidth: read + write bytes of a device-to-device copy."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def ssd_prefill_bench(torch, B, layer, u, out, stream, w, steps, warmup, ms_sequential):
    """The same layer prefill with the chunked (SSD-form) scan variant.  Its
    contract differs from the method's (no per-step rounding of the state), so
    it is reported beside the headline, never as it.  Roofline: the three chunk
    kernels are float64 multiply-add bound; per (batch, head, chunk of Q = 64):
    2 Q P N (chunk state) + 2 Q Q P (within the chunk) + 2 Q N P (from the
    entering state) + 2 P N (across chunks) flops."""
    s = w.shape
    for _ in range(warmup):
        layer.prefill(u, out, stream=stream, scan="ssd")
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    opts = [B.layer_opts(events=[None, None, None, a, b, None, None]) for a, b in evs]
    t0 = time.perf_counter()
    for i in range(steps):
        layer.prefill(u, out, stream=stream, scan="ssd", opts=opts[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    scan_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    Q, P, N = 64, s.headdim, s.dstate
    nc = (w.seqlen + Q - 1) // Q
    flops = w.batch * s.nheads * nc * (2 * Q * P * N + 2 * Q * Q * P + 2 * Q * N * P + 2 * P * N)
    achieved = flops / (scan_ms / 1e3) / 1e12
    return {"value": round(w.tokens / (ms / 1e3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms, 4), "scan_ms": round(scan_ms, 4),
            "speedup_vs_sequential": round(ms_sequential / ms, 3),
            "contract": "scan without per-step state rounding (float64): y within 1 of the "
                        "correctly rounded real recurrence",
            "roofline": {"bound": "fp64", "kernel": "ssd_chunk_*_kernel",
                         "achieved": round(achieved, 3), "peak": FP64_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / FP64_PEAK_TFLOPS, 4),
                         "work": f"{flops} flops per call"}}


def decode_bench(torch, configs, synth, stack=None, warmup=8, max_steps=None,
                 narrow_bits=(16, 24)):
    """Decode tokens/s of the 64-layer 2.7B-shaped stack, batch 16.

    A 1024-token seeding prefill fills the caches; then the workload's 512 one-token
    steps run as replays of one captured graph (every layer of a step): `warmup`
    untimed, the rest timed with HIP events.  Roofline: HBM, with the algorithmic
    bytes of a layer step = SSM state read + written + both int8 weight matrices +
    the conv window read + written.  The int32 state is the method's; the same
    stack then runs again from a fresh seeding prefill with each narrow state
    width in `narrow_bits` (codes on a per-layer power-of-two grid)."""
    import numpy as np
    from quantized_state_space_fwht_amd.runtime import DecodeGraph, Mamba2Stack
    w = configs.get(DECODE_WORKLOAD)
    s = w.shape
    if stack is None:
        log(f"bench: building decode stack {w.name} ({w.description})")
        stack = Mamba2Stack(s, (synth.workload_params(w, l) for l in range(w.nlayers)))
    else:
        log(f"bench: decode {w.name} on the same weights ({w.description})")
    u0 = torch.from_numpy(synth.workload_activations(w)).cuda()
    nsteps = w.decode_steps if max_steps is None else min(w.decode_steps, warmup + max_steps)
    inputs = torch.from_numpy(np.stack([synth.decode_step_input(w, t)
                                        for t in range(nsteps)])).cuda()
    weight_b = s.d_in_proj * s.d_model + s.d_model * s.d_inner
    conv_b = 2 * w.batch * s.conv_ch * 3

    def run(bits):
        stack.prefill(u0, with_cache=True)
        shifts = stack.narrow_states(bits) if bits != 32 else None
        g = DecodeGraph(stack, w.batch)
        for t in range(warmup):
            g.step(inputs[t])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(warmup, nsteps):
            g.step(inputs[t])
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (nsteps - warmup)
        state_b = 2 * w.batch * s.nheads * s.headdim * s.dstate * bits // 8
        step_bytes = w.nlayers * (state_b + weight_b + conv_b)
        gbs = step_bytes / (ms / 1e3) / 1e9
        res = {"value": round(w.batch / (ms / 1e3), 1), "unit": "tokens/s",
               "ms_per_token_step": round(ms, 4),
               "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                            "bytes_per_token_step": step_bytes}}
        if shifts is not None:
            res["state_shift_range"] = [min(shifts), max(shifts)]
        g.close()
        del g
        return res

    out = {"workload": w.name, **run(32), "batch": w.batch, "layers": w.nlayers,
           "steps_timed": nsteps - warmup, "steps_warmup": warmup, "seeding_prefill": w.seqlen,
           "state": "int32"}
    out["narrow_state"] = {f"int{b}": run(b) for b in narrow_bits}
    return out


def study_state(torch, configs, synth, B, steps=128):
    """Narrow decode-state caches: accuracy against the int32 state over decode steps.

    The 64-layer 2.7B-shaped stack (batch 16) is seeded by the same 1024-token
    prefill, then decodes the same `steps` tokens with the int32 state, 24-bit
    and 16-bit codes (each layer's shift chosen from its prefill state with one
    bit of headroom), and, as a control, with the int32 state and every decode
    input scaled by (1 + 2^-20).  Reported per step: the relative L2 error of the stack's
    contribution h_t - u_t against the int32 run; after the last step, for layers
    0, 31 and 63, the relative L2 error of the widened state and the share of
    codes at the saturation limits; the relative L2 error of layer 0's mixer output,
    whose input is the same in every run, isolates the format's own error from
    its propagation through the stack.  The oracle beside recomputes a 2.7B-shaped
    layer from an 8-token prefill through three 16-bit decode steps."""
    import numpy as np
    import oracle as O
    from quantized_state_space_fwht_amd.runtime import Mamba2Layer, Mamba2Stack
    w = configs.get(DECODE_WORKLOAD)
    s = w.shape
    log(f"study: building {w.name} ({w.description})")
    stack = Mamba2Stack(s, (synth.workload_params(w, l) for l in range(w.nlayers)))
    u0 = torch.from_numpy(synth.workload_activations(w)).cuda()
    inputs = torch.from_numpy(np.stack([synth.decode_step_input(w, t)
                                        for t in range(steps)])).cuda()
    probe_layers = (0, w.nlayers // 2 - 1, w.nlayers - 1)
    runs = {}
    # "ctl": the int32 state with every decode input scaled by (1 + 2^-20), the
    # stack's own sensitivity to a perturbation far below any state rounding
    for bits in (32, 24, 16, "ctl"):
        stack.prefill(u0, with_cache=True)
        shifts = stack.narrow_states(bits) if bits in (16, 24) else [0] * w.nlayers
        xs = inputs * (1.0 + 2.0 ** -20) if bits == "ctl" else inputs
        contrib, mix0 = [], []
        t0 = time.perf_counter()
        for t in range(steps):
            h = xs[t].contiguous()
            for l, layer in enumerate(stack.layers):
                nxt = layer.decode(h)
                if l == 0:
                    mix0.append((nxt - h).double())  # layer 0: the same input in every run
                h = nxt
            contrib.append((h - xs[t]).double())
        torch.cuda.synchronize()
        sec = time.perf_counter() - t0
        states, sat = {}, {}
        for l in probe_layers:
            layer = stack.layers[l]
            st = layer.wide_state() if bits in (16, 24) else layer.cache_t["ssm_state"]
            states[l] = st.double()
            if bits in (16, 24):
                lim = (1 << (bits - 1))
                c = torch.div(st.long(), 1 << shifts[l], rounding_mode="floor")
                sat[l] = float(((c == lim - 1) | (c == -lim)).double().mean().item())
        runs[bits] = {"contrib": torch.stack(contrib), "mix0": torch.stack(mix0),
                      "states": states, "sat": sat,
                      "shifts": shifts, "sec": sec}
        log(f"study: {bits} done ({sec:.1f} s eager)")
    ref = runs[32]
    report = {"study": "narrow_state", "workload": w.name, "steps": steps,
              "seeding_prefill": w.seqlen, "batch": w.batch, "layers": w.nlayers, "widths": {}}
    marks = [t for t in (0, 1, 7, 31, 63, steps - 1) if t < steps]
    for bits in (24, 16, "ctl"):
        r = runs[bits]
        d = r["contrib"] - ref["contrib"]
        rel = (d.flatten(1).norm(dim=1) / ref["contrib"].flatten(1).norm(dim=1)).cpu().numpy()
        d0 = r["mix0"] - ref["mix0"]
        rel0 = (d0.flatten(1).norm(dim=1) / ref["mix0"].flatten(1).norm(dim=1)).cpu().numpy()
        report["widths"]["int32_input_x(1+2^-20)" if bits == "ctl" else f"int{bits}"] = {
            "shift_min": min(r["shifts"]), "shift_max": max(r["shifts"]),
            "shift_mean": round(float(np.mean(r["shifts"])), 2),
            "contrib_rel_l2_at_step": {str(t + 1): float(rel[t]) for t in marks},
            "contrib_rel_l2_max": float(rel.max()),
            "layer0_out_rel_l2_at_step": {str(t + 1): float(rel0[t]) for t in marks},
            "layer0_out_rel_l2_max": float(rel0.max()),
            "state_rel_l2_after": {str(l): float(((r["states"][l] - ref["states"][l]).norm()
                                                  / ref["states"][l].norm()).item())
                                   for l in probe_layers},
            "saturated_code_share_after": {str(l): r["sat"].get(l, 0.0) for l in probe_layers}}
    # the oracle beside: one 2.7B-shaped layer, 8-token prefill, three 16-bit steps
    wl = configs.with_len(w, w.batch, 11)
    params = synth.workload_params(wl, 0)
    u = synth.workload_activations(wl)
    t0 = time.perf_counter()
    prep = O.prepare_layer(params)
    _, _, cache, _ = O.layer_prefill(prep, s, u[:, :8])
    sh = O.state_shift_for(int(np.max(np.abs(cache["ssm_state"]))), 16)
    cache["ssm_state"] = O.narrow_state(cache["ssm_state"], 16, sh)
    want = []
    for t in range(8, 11):
        o, _, cache, _ = O.layer_decode(prep, s, u[:, t], cache, state_fmt=(16, sh))
        want.append(o)
    osec = time.perf_counter() - t0
    layer = Mamba2Layer(s, params)
    layer.prefill(torch.from_numpy(u[:, :8]).cuda())
    agree = layer.narrow_state(16) == sh
    for t, o in zip(range(8, 11), want):
        got = layer.decode(torch.from_numpy(np.ascontiguousarray(u[:, t])).cuda())
        agree = agree and bool(np.array_equal(got.cpu().numpy(), o))
    agree = agree and bool(np.array_equal(layer.cache_t["ssm_codes"].cpu().numpy(),
                                          O.pack_state(cache["ssm_state"], 16)))
    report["oracle_beside"] = {"sample": "one 2.7B-shaped layer, batch 16, 8-token prefill, "
                                         "three decode steps with 16-bit codes",
                               "seconds": round(osec, 2), "agrees": agree}
    return report


def study_scales(torch, configs, synth, B):
    """Static against dynamic scales on held-out inputs (the scale study).

    The 24-layer 130M-shaped static stack is calibrated on its 64 seeded
    sequences (one per call, as the oracle's calibration runs them), then its
    8 held-out sequences run once with the static scales and once with dynamic
    ones.  Per quantization point and layer the library reports the clip count
    and the dequantization error; this prints the clip rate and the SQNR
    (10 log10 of sum v^2 over sum (v - q step)^2).  Beside it, the oracle
    recomputes layer 0 in dynamic mode on the first held-out sequence, checked
    against the library's record of the same call and timed."""
    import numpy as np
    import oracle as O
    from quantized_state_space_fwht_amd.runtime import Mamba2Stack
    w = configs.get(STUDY_WORKLOAD)
    s = w.shape
    log(f"study: building {w.name} ({w.description})")
    params = [synth.workload_params(w, l) for l in range(w.nlayers)]
    stack = Mamba2Stack(s, params)
    calib = [torch.from_numpy(x).cuda() for x in synth.calibration_sequences(w)]
    t0 = time.perf_counter()
    stack.calibrate(calib)
    torch.cuda.synchronize()
    calib_s = time.perf_counter() - t0
    u = torch.from_numpy(synth.eval_batch(w)).cuda()
    rows = {}
    outs = {}
    for mode in ("static", "dynamic"):
        if mode == "dynamic":
            for layer in stack.layers:
                layer.set_dynamic()
        bufs = [B.quant_stats_buffer() for _ in stack.layers]
        outs[mode] = stack.prefill(u, with_cache=False, quant_stats=bufs).float().cpu().numpy()
        rows[mode] = [B.quant_stats_from_device(b) for b in bufs]
    # time the held-out pass with and without statistics (dynamic mode)
    def timed(with_stats):
        bufs = [B.quant_stats_buffer() for _ in stack.layers] if with_stats else None
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        stack.prefill(u, with_cache=False, quant_stats=bufs)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)
    timed(False)
    ms_plain, ms_stats = timed(False), timed(True)

    def summary(recs):
        out = {}
        for i, name in enumerate(B.QP_NAMES):
            cnt = sum(r.count[i] for r in recs)
            clip = sum(r.clipped[i] for r in recs)
            se = sum(r.sq_err[i] for r in recs)
            sv = sum(r.sq_val[i] for r in recs)
            per_layer_db = [round(10 * np.log10(r.sq_val[i] / r.sq_err[i]), 2) if r.sq_err[i] > 0
                            else None for r in recs]
            out[name] = {"clip_rate": clip / cnt if cnt else 0.0, "clipped": int(clip),
                         "elements": int(cnt),
                         "sqnr_db": round(10 * np.log10(sv / se), 3) if se > 0 else None,
                         "sqnr_db_per_layer": per_layer_db,
                         "clipped_per_layer": [int(r.clipped[i]) for r in recs]}
        return out
    diff = outs["static"] - outs["dynamic"]
    rel_l2 = float(np.linalg.norm(diff) / np.linalg.norm(outs["dynamic"]))

    # the oracle beside: layer 0, dynamic, first held-out sequence
    log("study: oracle check (layer 0, dynamic, one held-out sequence)")
    u0 = synth.eval_batch(w)[:1]
    xin = O.rmsnorm_fixed_order(u0.reshape(-1, s.d_model),
                                np.ones(s.d_model, np.float32)).reshape(u0.shape)
    t0 = time.perf_counter()
    _, r, _, _ = O.layer_prefill(O.prepare_layer(params[0]), s, xin, "dynamic", collect=True)
    oracle_s = time.perf_counter() - t0
    buf = B.quant_stats_buffer()
    stack.layers[0].set_dynamic()
    # the stack's layers apply the pre-norm themselves: they take u itself
    stack.layers[0].prefill(torch.from_numpy(np.ascontiguousarray(u0)).cuda(),
                            with_cache=False, opts=B.layer_opts(quant_stats=buf))
    torch.cuda.synchronize()
    g = B.quant_stats_from_device(buf)
    agree = all(g.count[i] == r["qstats"][n]["count"] and g.clipped[i] == r["qstats"][n]["clipped"]
                and abs(g.sq_err[i] - r["qstats"][n]["sq_err"]) <= 1e-9 * r["qstats"][n]["sq_err"]
                for i, n in enumerate(B.QP_NAMES))
    return {"study": "static_vs_dynamic_scales", "workload": w.name, "layers": w.nlayers,
            "calibration": f"{len(w.calib_seeds)} sequences x {w.seqlen} tokens (seeds "
                           f"{w.calib_seeds[0]}-{w.calib_seeds[-1]})",
            "held_out": f"{len(w.eval_seeds)} sequences x {w.seqlen} tokens (seeds "
                        f"{w.eval_seeds[0]}-{w.eval_seeds[-1]})",
            "static": summary(rows["static"]), "dynamic": summary(rows["dynamic"]),
            "output_rel_l2_static_vs_dynamic": rel_l2,
            "gpu": {"calibration_s": round(calib_s, 3), "held_out_pass_ms": round(ms_plain, 3),
                    "held_out_pass_with_stats_ms": round(ms_stats, 3)},
            "oracle_beside": {"sample": "layer 0, dynamic, held-out sequence 0 (2048 tokens)",
                              "seconds": round(oracle_s, 2), "agrees": bool(agree)}}


def study_outliers(torch, configs, synth, B, rows=2048):
    """The outlier study: Hadamard against plain per-tensor and smoothed W8A8.

    For the in_proj and out_proj of one 130M-shaped and one 2.7B-shaped layer
    (their inputs: the synthetic activations with four outlier channels at 50x,
    and the normed gate output of a dynamic layer pass over them; the first
    `rows` tokens), each scheme runs on the GPU (quantization, int8 GEMM,
    dequantization) and is compared with the float64 product on the host:
    output error ||out - x w^T|| / ||x w^T|| and the activation SQNR in the
    scheme's own domain.  The oracle recomputes the 130M in_proj beside."""
    import numpy as np
    import oracle as O
    from quantized_state_space_fwht_amd.runtime import Mamba2Layer

    def gpu_scheme(xd, wd, name):
        n, k = wd.shape
        m = xd.shape[0]
        qa = torch.empty((m, k), dtype=torch.int8, device="cuda")
        qb = torch.empty((n, k), dtype=torch.int8, device="cuda")
        sa = torch.empty(1, dtype=torch.float32, device="cuda")
        sb = torch.empty(1, dtype=torch.float32, device="cuda")
        xs = xd
        if name == "hadamard":
            B.fm_hadamard_quant(xd, B.DYNAMIC, 0, 0, qa, sa)
            B.fm_hadamard_quant(wd, B.DYNAMIC, 0, 0, qb, sb)
        elif name == "naive":
            B.fm_quant_per_tensor(xd, qa, sa)
            B.fm_quant_per_tensor(wd, qb, sb)
        else:
            s = torch.empty(k, dtype=torch.float32, device="cuda")
            B.fm_smooth_scales(xd, wd, s)
            xs = torch.empty_like(xd)
            ws = torch.empty_like(wd)
            B.fm_scale_columns(xd, s, True, xs)
            B.fm_scale_columns(wd, s, False, ws)
            B.fm_quant_per_tensor(xs, qa, sa)
            B.fm_quant_per_tensor(ws, qb, sb)
        out = torch.empty((m, n), dtype=torch.float32, device="cuda")
        B.fm_w8a8_gemm(qa, qb, sa, sb, out=out)
        return qa, sa, xs, out

    import scipy.linalg
    h256 = scipy.linalg.hadamard(256).astype(np.float64) / 16.0  # symmetric, orthonormal
    report = {"study": "outlier_schemes", "rows": rows, "layers": {}}
    for wl in ("m130m_layer", "m2p7b_stack"):
        w = configs.get(wl)
        s = w.shape
        params = synth.workload_params(w, 0)
        u = synth.workload_activations(configs.with_len(w, batch=1, seqlen=rows))
        layer = Mamba2Layer(s, params)
        layer.prefill(torch.from_numpy(u).cuda(), opts=B.layer_opts(keep=True))
        normed = layer.tap("normed", torch.float32, (rows, s.d_inner)).clone()
        cases = {"in_proj": (u.reshape(rows, s.d_model), params["w_in"]),
                 "out_proj": (normed.cpu().numpy(), params["w_out"])}
        for lname, (x, wt) in cases.items():
            x = np.ascontiguousarray(x, np.float32)
            wt = np.ascontiguousarray(wt, np.float32)
            ref = x.astype(np.float64) @ wt.astype(np.float64).T
            nref = np.linalg.norm(ref)
            xd, wd = torch.from_numpy(x).cuda(), torch.from_numpy(wt).cuda()
            entry = {"m": x.shape[0], "k": x.shape[1], "n": wt.shape[0], "schemes": {}}
            for sch in ("hadamard", "naive", "smooth"):
                gpu_scheme(xd, wd, sch)  # warm
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                qa, sa, xs, out = gpu_scheme(xd, wd, sch)
                torch.cuda.synchronize()
                ms = (time.perf_counter() - t0) * 1e3
                o = out.cpu().numpy().astype(np.float64)
                if sch == "hadamard":  # the rotated activations (exact, float64), for the SQNR
                    xs_h = (x.astype(np.float64).reshape(-1, 256) @ h256).reshape(x.shape)
                else:
                    xs_h = xs.cpu().numpy().astype(np.float64)
                e = xs_h - qa.cpu().numpy().astype(np.float64) * float(sa.item())
                entry["schemes"][sch] = {
                    "output_rel_err": float(np.linalg.norm(o - ref) / nref),
                    "activation_sqnr_db": float(10 * np.log10(np.sum(xs_h ** 2) / np.sum(e * e))),
                    "gpu_ms": round(ms, 3)}
            report["layers"][f"{wl}.{lname}"] = entry
        del layer
        torch.cuda.empty_cache()
    # the oracle beside: the 130M in_proj, all three schemes
    w = configs.get("m130m_layer")
    params = synth.workload_params(w, 0)
    x = synth.workload_activations(configs.with_len(w, batch=1, seqlen=rows)).reshape(rows, -1)
    t0 = time.perf_counter()
    errs = {sch: O.outliers.output_error(O.outliers.scheme(x, params["w_in"], sch)["out"], x,
                                         params["w_in"]) for sch in ("hadamard", "naive", "smooth")}
    osec = time.perf_counter() - t0
    got = report["layers"]["m130m_layer.in_proj"]["schemes"]
    report["oracle_beside"] = {"sample": f"m130m_layer in_proj, {rows} tokens, three schemes",
                               "seconds": round(osec, 2),
                               "agrees": all(errs[k] == got[k]["output_rel_err"] for k in errs)}
    return report


def study_nau(torch, configs, synth, B):
    """Alternative coefficient tables for the 8-segment 2^v unit.

    The pages fix the unit's form (first-order segments on the eighths of an
    octave) but not its coefficients.  For the chord table, a least-squares and
    a minimax (relative error) fit of the same form, the library evaluates exp
    on every Q.16 input in [-16, 0] and SoftPlus, SiLU on every input in
    [-16, 16]; the host compares with the exact functions (float64): largest
    and RMS error in units of 2^-16.  The oracle recomputes a sample beside."""
    import numpy as np
    import oracle as O
    tables = synth.nau_knot_tables()
    span = 16 << 16
    xs = {"exp": np.arange(-span, 1, dtype=np.int64),
          "softplus": np.arange(-span, span + 1, dtype=np.int64),
          "silu": np.arange(-span, span + 1, dtype=np.int64)}
    exact = {"exp": lambda x: np.exp(x / 65536.0) * 65536.0,
             "softplus": lambda x: np.logaddexp(0.0, x / 65536.0) * 65536.0,
             "silu": lambda x: (x / 65536.0) / (1.0 + np.exp(-x / 65536.0)) * 65536.0}
    # the unit's own form with an exact exponential: SoftPlus is e^-|x| + max(x, 0)
    # (Eq. (5) and the symmetry), whose gap to ln(1 + e^x) no table can close
    form = {"exp": exact["exp"],
            "softplus": lambda x: (np.exp(-np.abs(x) / 65536.0) + np.maximum(x, 0) / 65536.0)
            * 65536.0,
            "silu": exact["silu"]}
    codes = {"exp": B.NAU_EXP, "softplus": B.NAU_SOFTPLUS, "silu": B.NAU_SILU}
    report = {"study": "nau_knot_tables", "domain": "all Q.16 inputs, exp on [-16, 0], "
              "SoftPlus and SiLU on [-16, 16]", "tables": {}}
    for name, knots in tables.items():
        entry = {"knots_q30": [int(v) for v in knots]}
        for fn, x in xs.items():
            xd = torch.from_numpy(x.astype(np.int32)).cuda()
            yd = torch.empty_like(xd)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            B.fm_nau_eval_knots(codes[fn], knots, xd, yd)
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) * 1e6
            got = yd.cpu().numpy().astype(np.float64)
            err = got - exact[fn](x.astype(np.float64))
            ferr = got - form[fn](x.astype(np.float64))
            entry[fn] = {"max_abs_lsb": float(np.max(np.abs(err))),
                         "rms_lsb": float(np.sqrt(np.mean(err * err))),
                         "mean_lsb": float(np.mean(err)),
                         "vs_form_max_abs_lsb": float(np.max(np.abs(ferr))),
                         "vs_form_rms_lsb": float(np.sqrt(np.mean(ferr * ferr))),
                         "gpu_us": round(us, 1)}
        # largest relative error of 2^f itself (the form's accuracy), over all fractions
        k = np.arange(1 << 16)
        y = knots.astype(np.float64) / 2 ** 30
        seg, r = k >> 13, (k & 8191) / 8192.0
        rel = (y[seg] * (1 - r) + y[seg + 1] * r) / 2.0 ** (k / 65536.0) - 1
        entry["exp2_max_rel"] = float(np.max(np.abs(rel)))
        report["tables"][name] = entry
    # the oracle beside: exp with the minimax table on a strided sample
    x = np.arange(-span, 1, 31, dtype=np.int64)
    t0 = time.perf_counter()
    want = O.exp_q16(x, tables["minimax"])
    osec = time.perf_counter() - t0
    xd = torch.from_numpy(x.astype(np.int32)).cuda()
    yd = torch.empty_like(xd)
    B.fm_nau_eval_knots(B.NAU_EXP, tables["minimax"], xd, yd)
    report["oracle_beside"] = {"sample": f"exp, minimax table, {x.size} inputs",
                               "seconds": round(osec, 3),
                               "agrees": bool(np.array_equal(yd.cpu().numpy(), want))}
    return report


def stage_work(s, T):
    """Algorithmic work of each stage of one layer call over T tokens, with the
    roofline that bounds it: (bound, amount, unit of the amount, what counts).
    The stage boundaries are the library's stage events (fm_layer_opts)."""
    dm, di, N, H, P = s.d_model, s.d_inner, s.dstate, s.nheads, s.headdim
    ch, dip = di + 2 * N, 2 * di + 2 * N + H
    return {
        "in_quant": ("hbm", 5 * T * dm, "B", "4 B read + 1 B code written per in_proj input "
                                              "element (rotation, maximum, codes)"),
        "in_proj": ("mfma", 2 * T * dip * dm, "op", "2 M N K int8 operations"),
        "conv": ("hbm", T * (5 * ch + 12 * H), "B",
                 "4 B float read + 1 B code written per xBC element; 4 B read + 8 B written "
                 "per (token, head) for dt and the decay"),
        "scan": ("alu", SCAN_OPS_PER_ELEMENT_STEP * T * H * P * N, "op",
                 "8 integer operations per state element and step"),
        "gate_quant": ("hbm", 9 * T * di, "B", "4 B y + 4 B z read + 1 B code written per "
                                               "out_proj input element"),
        "out_proj": ("mfma", 2 * T * dm * di, "op", "2 M N K int8 operations"),
    }


def stage_report(s, T, ms):
    """Per stage: average milliseconds per layer call and its roofline fraction."""
    peaks = {"hbm": (HBM_PEAK_GBS, "GB/s", 1e9), "mfma": (I8_MFMA_PEAK_TOPS, "TOP/s", 1e12),
             "alu": (VALU_PEAK_TOPS, "TOP/s", 1e12)}
    out = {}
    for name, (bound, amount, _, what) in stage_work(s, T).items():
        peak, unit, scale = peaks[bound]
        t = ms[name]
        ach = amount / (t / 1e3) / scale if t > 0 else 0.0
        out[name] = {"ms": round(t, 4), "bound": bound, "achieved": round(ach, 1), "peak": peak,
                     "unit": unit, "frac": round(ach / peak, 4), "work_per_call": amount,
                     "work": what}
    return out


class Model:
    """The workload's layers on the GPU: one bare layer, or a pre-norm residual
    stack (static stacks calibrated on their seeded calibration sequences)."""

    def __init__(self, torch, configs, synth, w):
        from quantized_state_space_fwht_amd.runtime import Mamba2Layer, Mamba2Stack
        self.w = w
        if w.nlayers == 1:
            self.layers = [Mamba2Layer(w.shape, synth.workload_params(w, 0))]
            self.stack = None
        else:
            self.stack = Mamba2Stack(w.shape, (synth.workload_params(w, l)
                                               for l in range(w.nlayers)), mode="dynamic")
            self.layers = self.stack.layers
            if w.mode == "static":
                log(f"bench: calibrating {w.name} on {len(w.calib_seeds)} sequences")
                self.stack.calibrate([torch.from_numpy(x).cuda()
                                      for x in synth.calibration_sequences(w)])
        u = synth.eval_batch(w) if w.mode == "static" else synth.workload_activations(w)
        self.u = torch.from_numpy(u).cuda()
        self.bufs = [torch.empty_like(self.u), torch.empty_like(self.u)]

    def step(self, stream, opts=None):
        """One prefill pass; opts: None or one LayerOpts per layer."""
        if self.stack is None:
            self.layers[0].prefill(self.u, self.bufs[0], stream=stream,
                                   opts=None if opts is None else opts[0])
            return self.bufs[0]
        return self.stack.prefill(self.u, with_cache=True, stream=stream, layer_opts=opts,
                                  bufs=self.bufs)


def prefill_bench(torch, B, model, steps, warmup):
    """Time `steps` prefill passes after `warmup`; the scan kernel of every layer
    is bracketed by HIP events on its stream; then one more pass with every
    stage boundary recorded gives the per-stage times."""
    w, s = model.w, model.w.shape
    stream = torch.cuda.current_stream()
    nl = len(model.layers)
    for _ in range(warmup):
        model.step(stream)
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    scan_evs = [[(ev(), ev()) for _ in range(nl)] for _ in range(steps)]
    for row in scan_evs:  # create the underlying HIP events outside the timed region
        for a, b in row:
            a.record(stream)
            b.record(stream)
    opts = [[B.layer_opts(events=[None, None, None, a, b, None, None]) for a, b in row]
            for row in scan_evs]
    torch.cuda.synchronize()
    log(f"bench: timing {steps} steps of {w.name}")
    t0 = time.perf_counter()
    for i in range(steps):
        model.step(stream, opts[i])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    scan_ms = sum(a.elapsed_time(b) for row in scan_evs for a, b in row) / (steps * nl)
    # the stage breakdown: one more pass, every boundary of every layer recorded
    stage_evs = [[ev() for _ in range(B.LAYER_EVENTS)] for _ in range(nl)]
    for row in stage_evs:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    model.step(stream, [B.layer_opts(events=row) for row in stage_evs])
    torch.cuda.synchronize()
    stage_ms = {name: sum(row[k].elapsed_time(row[k + 1]) for row in stage_evs) / nl
                for k, name in enumerate(B.STAGES)}
    T = w.batch * w.seqlen
    elem_steps = T * s.nheads * s.headdim * s.dstate
    achieved = SCAN_OPS_PER_ELEMENT_STEP * elem_steps / (scan_ms / 1e3) / 1e12
    roofline = {"bound": "alu", "kernel": "scan_kernel", "achieved": round(achieved, 3),
                "peak": round(VALU_PEAK_TOPS, 2), "unit": "TOP/s",
                "frac": round(achieved / VALU_PEAK_TOPS, 4),
                "traffic": load_traffic(w.name, elem_steps),
                "launch_ms": round(scan_ms, 4), "launches_timed": steps * nl,
                "work": f"{SCAN_OPS_PER_ELEMENT_STEP} ops x {elem_steps} element-steps per launch"}
    return {"value": round(w.tokens / (ms_per_step / 1e3), 1), "ms_per_step": ms_per_step,
            "roofline": roofline, "stages": stage_report(s, T, stage_ms),
            "stage_ms_sum_per_layer": round(sum(stage_ms.values()), 4)}


def workload_config(w):
    s = w.shape
    return {"workload": w.name, "layers": w.nlayers, "batch": w.batch, "seq_len": w.seqlen,
            "d_model": s.d_model, "d_inner": s.d_inner, "nheads": s.nheads,
            "headdim": s.headdim, "d_state": s.dstate, "mode": w.mode,
            "parallelism": "single-gpu"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=HEADLINE_WORKLOAD,
                    help="prefill workload timed for the headline (default: the 64-layer "
                         "2.7B-shaped stack, batch 4, L 4096)")
    ap.add_argument("--layers", type=int, default=None,
                    help="run only the first N layers of a stack workload (every layer runs the "
                         "same kernels at the same shapes: for profiler runs); config.layers "
                         "then says N")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline workload (no 130M layer / static stack / "
                         "decode / chunked-scan lines)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode measurement (64-layer 2.7B-shaped stack)")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="time only this many decode steps (default: the workload's)")
    ap.add_argument("--study-scales", action="store_true",
                    help="run the static-vs-dynamic scale study instead of the benchmark "
                         "(one JSON line of clip rates and SQNR per quantization point)")
    ap.add_argument("--study-outliers", action="store_true",
                    help="run the outlier study (Hadamard against plain per-tensor and smoothed "
                         "W8A8 on the projections' inputs) instead of the benchmark")
    ap.add_argument("--study-state", action="store_true",
                    help="run the narrow decode-state accuracy study (int32 against 24- and "
                         "16-bit codes on the 2.7B-shaped stack) instead of the benchmark")
    ap.add_argument("--study-nau", action="store_true",
                    help="run the 2^v unit's coefficient study (chord, least-squares and "
                         "minimax tables) instead of the benchmark")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, copy 256 MiB device-to-device three times "
                         "(a reference kernel of known traffic for counter runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (the layer would "
              "shard over the batch); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_state_space_fwht_amd import binding as B
    from quantized_state_space_fwht_amd import configs, synth

    if args.study_scales:
        torch.cuda.set_device(0)
        print(json.dumps(study_scales(torch, configs, synth, B)), flush=True)
        return
    if args.study_state:
        torch.cuda.set_device(0)
        print(json.dumps(study_state(torch, configs, synth, B)), flush=True)
        return
    if args.study_nau:
        torch.cuda.set_device(0)
        print(json.dumps(study_nau(torch, configs, synth, B)), flush=True)
        return
    if args.study_outliers:
        torch.cuda.set_device(0)
        print(json.dumps(study_outliers(torch, configs, synth, B)), flush=True)
        return

    w = configs.get(args.workload)
    if args.layers is not None:
        import dataclasses
        w = dataclasses.replace(w, nlayers=max(1, min(args.layers, w.nlayers)))
    if w.decode_steps:
        print("bench.py times prefill workloads (decode is an extra key)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    log(f"bench: building {w.name} ({w.description})")
    model = Model(torch, configs, synth, w)
    r = prefill_bench(torch, B, model, args.steps, args.warmup)
    line = {
        "metric": METRIC, "value": r["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8+int32", "data": "synthetic (seeded; random-init weights)",
        "config": workload_config(w), "roofline": r["roofline"], "stages": r["stages"],
        "stage_ms_sum_per_layer": r["stage_ms_sum_per_layer"],
    }
    extras = not args.no_extras
    if (extras and not args.no_decode and w.name == HEADLINE_WORKLOAD
            and w.nlayers == configs.get(DECODE_WORKLOAD).nlayers):
        # the decode workload has the same layer shapes and weights
        model.u = model.bufs = None
        torch.cuda.empty_cache()
        line["decode"] = decode_bench(torch, configs, synth, stack=model.stack,
                                      max_steps=args.decode_steps)
    del model
    torch.cuda.empty_cache()
    if extras:
        for name in ("m130m_layer", "m130m_stack_static"):
            if name == w.name:
                continue
            wx = configs.get(name)
            log(f"bench: building {wx.name} ({wx.description})")
            mx = Model(torch, configs, synth, wx)
            steps = 20 if wx.nlayers == 1 else 5
            rx = prefill_bench(torch, B, mx, steps, 3)
            line[name] = {"value": rx["value"], "unit": "tokens/s",
                          "ms_per_step": round(rx["ms_per_step"], 4), "steps": steps,
                          "config": workload_config(wx), "roofline": rx["roofline"],
                          "stages": rx["stages"]}
            if wx.nlayers == 1:
                stream = torch.cuda.current_stream()
                line[name]["prefill_ssd"] = ssd_prefill_bench(
                    torch, B, mx.layers[0], mx.u, mx.bufs[0], stream, wx, steps, 3,
                    rx["ms_per_step"])
            del mx
            torch.cuda.empty_cache()
    # the achievable HBM rate on this machine: a device-to-device copy of 512 MiB
    hbm_meas = measured_copy_gbs(torch)
    line["measured_peaks"] = {"hbm_copy_GBs": round(hbm_meas, 1),
                              "how": "512 MiB device-to-device copy, 10 timed, 2 x bytes"}
    if "decode" in line:
        for rr in [line["decode"]["roofline"]] + [v["roofline"] for v in
                                                  line["decode"].get("narrow_state", {}).values()]:
            rr["frac_of_measured"] = round(rr["achieved"] / hbm_meas, 4)
    if args.copy_probe:
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
