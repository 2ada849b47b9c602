"""Quantization statistics (clip counts, dequantization error) against the oracle.

The library adds, for each of a layer's six activation quantization points,
the number of elements, how many codes were clamped, the sum of squared
dequantization errors and the sum of squared values into a device record
(fm_quant_stats, requested per call through fm_layer_opts.quant_stats).  Counts must equal
the oracle's exactly; the float64 sums are added atomically in a varying
order, so they are compared within 1e-9 relative.
"""
import numpy as np
import pytest

import oracle as O
from quantized_state_space_fwht_amd import configs, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).cuda().contiguous()


def check_point_stats(got, want, where):
    from quantized_state_space_fwht_amd import binding as B
    for i, name in enumerate(B.QP_NAMES):
        w = want[name]
        assert got.count[i] == w["count"], (where, name, "count", got.count[i], w["count"])
        assert got.clipped[i] == w["clipped"], (where, name, "clipped", got.clipped[i], w["clipped"])
        for field in ("sq_err", "sq_val"):
            g, o = getattr(got, field)[i], w[field]
            assert g == pytest.approx(o, rel=1e-9, abs=1e-300), (where, name, field, g, o)


@pytest.mark.parametrize("wl,batch,seqlen", [("tiny_layer", 2, 40), ("m130m_layer", 1, 96)])
def test_layer_stats_dynamic(wl, batch, seqlen):
    from quantized_state_space_fwht_amd import binding as B
    from quantized_state_space_fwht_amd.runtime import Mamba2Layer
    w = configs.with_len(configs.get(wl), batch=batch, seqlen=seqlen)
    params = synth.workload_params(w, 0)
    u = synth.workload_activations(w)
    _, r, _, _ = O.layer_prefill(O.prepare_layer(params), w.shape, u, collect=True)
    layer = Mamba2Layer(w.shape, params)
    buf = B.quant_stats_buffer()
    layer.prefill(dev(u), opts=B.layer_opts(quant_stats=buf))
    torch.cuda.synchronize()
    got = B.quant_stats_from_device(buf)
    check_point_stats(got, r["qstats"], wl)
    assert sum(got.clipped) == 0  # dynamic scales never clip


def test_stack_stats_static_held_out():
    """Static scales calibrated on one short sequence, applied to held-out
    sequences: the Hadamard points clip; per layer and point the device record
    equals the oracle's."""
    from quantized_state_space_fwht_amd import binding as B
    from quantized_state_space_fwht_amd.runtime import Mamba2Stack
    w = configs.with_len(configs.get("tiny_layer"), batch=1, seqlen=48)
    params = [synth.workload_params(w, l) for l in range(3)]
    preps = [O.prepare_layer(p) for p in params]
    calib = synth.workload_activations(w, seed=100)
    qps, _ = O.calibrate_stack(preps, w.shape, [calib])
    w2 = configs.with_len(configs.get("tiny_layer"), batch=2, seqlen=64)
    u = synth.workload_activations(w2, seed=200)
    want = [O.quant_stats.empty() for _ in preps]
    O.stack_prefill(preps, w.shape, u, "static", qps, qstats=want)

    stack = Mamba2Stack(w.shape, params)
    stack.calibrate([dev(calib)])
    bufs = [B.quant_stats_buffer() for _ in params]
    stack.prefill(dev(u), quant_stats=bufs)
    torch.cuda.synchronize()
    total_clipped = 0
    for li, (buf, wl) in enumerate(zip(bufs, want)):
        got = B.quant_stats_from_device(buf)
        check_point_stats(got, wl, f"layer {li}")
        total_clipped += sum(got.clipped)
    assert total_clipped > 0


def test_collection_off_by_default_and_outputs_unchanged():
    """With collection on, the layer's outputs are the same bits as without."""
    from quantized_state_space_fwht_amd import binding as B
    from quantized_state_space_fwht_amd.runtime import Mamba2Layer
    w = configs.with_len(configs.get("tiny_layer"), batch=2, seqlen=33)
    params = synth.workload_params(w, 0)
    u = dev(synth.workload_activations(w))
    layer = Mamba2Layer(w.shape, params)
    ref = layer.prefill(u).clone()
    buf = B.quant_stats_buffer()
    got = layer.prefill(u, opts=B.layer_opts(quant_stats=buf)).clone()
    again = layer.prefill(u).clone()
    torch.cuda.synchronize()
    assert torch.equal(ref, got) and torch.equal(ref, again)
    assert B.quant_stats_from_device(buf).count[B.QP_U] > 0
