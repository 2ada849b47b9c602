"""The decode entry point that allocates nothing (fm_mamba2_layer_decode_noalloc)
against fm_mamba2_layer_decode with a caller workspace: outputs, caches and the
published record bit for bit, on consecutive calls whose second batch is smaller
(the shared scratch keeps the earlier call's contents)."""
import ctypes

import numpy as np
import pytest

from quantized_state_space_fwht_amd import configs, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).cuda().contiguous()


@pytest.mark.parametrize("wname,batches", [("m130m_layer", (65, 5)), ("m2p7b_stack", (16, 3))])
@pytest.mark.parametrize("mode", ["dynamic", "static"])
def test_decode_noalloc_equals_decode(wname, batches, mode):
    from quantized_state_space_fwht_amd import binding as B
    from quantized_state_space_fwht_amd.runtime import Mamba2Layer
    base = configs.get(wname)
    params = synth.workload_params(base, 0)
    stream = torch.cuda.current_stream()
    for batch in batches:
        w = configs.with_len(base, batch=batch, seqlen=24)
        s = w.shape
        u = synth.workload_activations(w, seed=batch)
        ref = Mamba2Layer(s, params, prenorm_residual=True)
        got = Mamba2Layer(s, params, prenorm_residual=True)
        if mode == "static":
            sp = B.StaticParams((1 << 14, 1 << 14), (13, 12), (3, 2, 3, 3))
            ref.set_static(sp)
            got.set_static(sp)
        ref.prefill(dev(u[:, :20]))
        got.prefill(dev(u[:, :20]))
        torch.cuda.synchronize()
        assert torch.equal(ref.cache_t["ssm_state"], got.cache_t["ssm_state"])
        for t in range(20, 24):
            x = dev(u[:, t])
            want = ref.decode(x)
            out = torch.empty_like(x)
            st = B.lib.fm_mamba2_layer_decode_noalloc(
                ctypes.byref(got.desc), ctypes.byref(got.weights),
                ctypes.byref(got.static) if got.static is not None else None, x.data_ptr(),
                batch, ctypes.byref(got.cache), out.data_ptr(), got.qp.data_ptr(), None,
                stream.cuda_stream)
            assert st == 0, B.lib.fm_last_error().decode()
            torch.cuda.synchronize()
            assert torch.equal(out, want), f"{wname} batch {batch} step {t}: output differs"
            for k in ("ssm_state", "conv_state", "p"):
                assert torch.equal(got.cache_t[k], ref.cache_t[k]), f"step {t}: {k} differs"
            assert torch.equal(got.qp, ref.qp), f"step {t}: published record differs"
