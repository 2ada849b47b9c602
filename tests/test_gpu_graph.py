"""A decode step of a stack captured as one HIP graph and replayed.

The library never allocates, synchronizes or clears memory with a copy
engine inside a call, so a whole decode step (every layer's launches) can be
captured on a stream and replayed.  Every replay, with eager work and host
synchronizations in between, must equal the eager decode of an identical
stack, outputs and caches bit for bit.
"""
import numpy as np
import pytest

from quantized_state_space_fwht_amd import configs, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).cuda().contiguous()


@pytest.mark.parametrize("mode", ["dynamic", "static"])
def test_decode_step_graph_replays_equal_eager(mode):
    from quantized_state_space_fwht_amd.runtime import DecodeGraph, Mamba2Stack
    w = configs.with_len(configs.get("m130m_stack_static"), batch=3, seqlen=40)
    s = w.shape
    params = [synth.workload_params(w, l) for l in range(3)]
    u = dev(synth.workload_activations(w, seed=200))
    eager, graphed = Mamba2Stack(s, params), Mamba2Stack(s, params)
    if mode == "static":
        calib = [dev(synth.workload_activations(w, seed=100))]
        eager.calibrate(calib)
        graphed.calibrate(calib)
    eager.prefill(u)
    graphed.prefill(u)
    g = DecodeGraph(graphed, w.batch)
    for t in range(6):
        x = dev(synth.decode_step_input(w, t))
        want = eager.decode(x)
        torch.cuda.synchronize()
        got = g.step(x)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"step {t}: graph output differs"
        for le, lg in zip(eager.layers, graphed.layers):
            for k in ("ssm_state", "conv_state", "p"):
                assert torch.equal(le.cache_t[k], lg.cache_t[k]), f"step {t}: {k} differs"
        # unrelated eager work and a host synchronization between replays
        _ = (u * 2).sum().item()


def test_graph_holds_its_buffers():
    """While a decode graph is open, a prefill that would replace its cache or
    grow its workspace raises and leaves the graph's buffers in place; the graph
    still replays correctly; after close() the prefill goes ahead."""
    from quantized_state_space_fwht_amd.runtime import DecodeGraph, GraphHeld, Mamba2Stack
    w = configs.with_len(configs.get("tiny_layer"), batch=2, seqlen=24)
    s = w.shape
    params = [synth.workload_params(w, l) for l in range(2)]
    u = dev(synth.workload_activations(w, seed=3))
    eager, graphed = Mamba2Stack(s, params), Mamba2Stack(s, params)
    eager.prefill(u)
    graphed.prefill(u)
    g = DecodeGraph(graphed, w.batch)
    u3 = dev(synth.workload_activations(configs.with_len(w, batch=3, seqlen=24), seed=4))
    with pytest.raises(GraphHeld):
        graphed.prefill(u3)                   # another batch: a new cache
    u_long = dev(synth.workload_activations(configs.with_len(w, batch=2, seqlen=4096), seed=5))
    with pytest.raises(GraphHeld):
        graphed.prefill(u_long)               # a larger workspace
    with pytest.raises(GraphHeld):
        graphed.narrow_states(16)
    for t in range(3):
        x = dev(synth.decode_step_input(w, t))
        want = eager.decode(x)
        got = g.step(x)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"step {t}"
    g.close()
    with pytest.raises(GraphHeld):
        g.step(x)
    graphed.prefill(u3)
    torch.cuda.synchronize()
    assert graphed.layers[0].cache_t["ssm_state"].shape[0] == 3
