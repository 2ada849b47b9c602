"""Host logic of the runtime's graph holds (CPU): while a captured decode graph
points at a stack's workspace and caches, nothing may replace them.

A captured graph replays raw device addresses, so a prefill with another batch
(a new cache), a larger workspace or a state narrowing would leave it reading
freed memory.  These checks run before any library call that computes, so they
are exercised here on CPU tensors without a GPU."""
import pytest
import torch

from quantized_state_space_fwht_amd import binding as B
from quantized_state_space_fwht_amd import configs
from quantized_state_space_fwht_amd.runtime import GraphHeld, Mamba2Layer, WorkspacePool


def _bare_layer(pool):
    """A layer object with its bookkeeping only (no weights are prepared)."""
    s = configs.get("tiny_layer").shape
    layer = Mamba2Layer.__new__(Mamba2Layer)
    layer.shape, layer.device = s, "cpu"
    layer.desc = B.LayerDesc(s.d_model, s.d_inner, s.nheads, s.headdim, s.dstate, s.d_conv,
                             B.DYNAMIC, 1)
    layer._pool, layer._ws, layer._ws_key = pool, None, None
    layer.cache, layer.ncache, layer.holds, layer.static = None, None, 0, None
    return layer


def test_pool_never_regrows_while_held():
    pool = WorkspacePool("cpu")
    t = pool.get(4096)
    pool.holds = 1
    assert pool.get(1024) is t and pool.get(4096) is t
    with pytest.raises(GraphHeld):
        pool.get(8192)
    assert pool.t is t
    pool.holds = 0
    assert pool.get(8192).numel() >= 8192


def test_layer_refuses_new_buffers_while_held():
    pool = WorkspacePool("cpu")
    layer = _bare_layer(pool)
    layer.workspace_for(2, 1)
    layer.alloc_cache(2)
    held = dict(layer.cache_t)
    layer.holds = 1
    pool.holds = 1
    with pytest.raises(GraphHeld):
        layer.alloc_cache(3)                          # a prefill with another batch
    with pytest.raises(GraphHeld):
        layer.prefill(torch.zeros(3, 4, layer.shape.d_model))
    with pytest.raises(GraphHeld):
        layer.workspace_for(2, 4096)                  # a prefill needing a larger workspace
    with pytest.raises(GraphHeld):
        layer.narrow_state(16, shift=0)
    assert all(layer.cache_t[k] is v for k, v in held.items())
    layer.holds = pool.holds = 0
    layer.alloc_cache(3)
    assert layer.cache_t["ssm_state"].shape[0] == 3
