"""Workload registry: the layer shapes and seeds of the five synthetic workloads.

Shapes follow the Mamba2 block (Fig. 2 of the FastMamba paper, "Computational
flow in Mamba2 block and SSM block"): in_proj produces [z | x | B | C | dt],
so its width is 2*d_inner + 2*d_state + nheads; the depthwise conv runs over
the x|B|C channels (d_inner + 2*d_state of them).  Block size 256 for the
Hadamard rotation is the block-diagonal reading of the paper's FindHadamard
step (Algorithm 1 in Section III-A leaves the construction open).

This module holds shapes and seeds only: no arithmetic of the method.
"""
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class LayerShape:
    d_model: int
    d_inner: int
    nheads: int
    headdim: int
    dstate: int
    d_conv: int = 4

    @property
    def conv_ch(self) -> int:
        return self.d_inner + 2 * self.dstate

    @property
    def d_in_proj(self) -> int:
        return 2 * self.d_inner + 2 * self.dstate + self.nheads

    def validate(self) -> None:
        assert self.nheads * self.headdim == self.d_inner
        assert self.d_model % 256 == 0 and self.d_inner % 256 == 0
        assert self.d_conv == 4


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    batch: int
    seqlen: int
    nlayers: int = 1
    mode: str = "dynamic"            # "dynamic" | "static"
    decode_steps: int = 0            # >0: one-token recurrent steps after a seeding prefill
    param_seed_base: int = 1000      # layer l draws its parameters from seed base + l
    input_seed: int = 0
    outlier_seed: int = 7
    n_outliers: int = 4
    outlier_scale: float = 50.0
    calib_seeds: tuple = ()          # static mode: sequences the scales are calibrated on
    eval_seeds: tuple = ()           # static mode: fresh sequences the scales are applied to
    description: str = ""

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


SHAPE_TINY = LayerShape(d_model=256, d_inner=512, nheads=8, headdim=64, dstate=64)
SHAPE_130M = LayerShape(d_model=768, d_inner=1536, nheads=24, headdim=64, dstate=128)
SHAPE_2P7B = LayerShape(d_model=2560, d_inner=5120, nheads=80, headdim=64, dstate=128)

WORKLOADS = {
    "tiny_layer": Workload(
        "tiny_layer", SHAPE_TINY, batch=1, seqlen=256,
        description="single mixer layer, d_model 256, batch 1, L 256 prefill"),
    "m130m_layer": Workload(
        "m130m_layer", SHAPE_130M, batch=1, seqlen=2048,
        description="one Mamba2-130M-shaped mixer layer, batch 1, L 2048 prefill"),
    "m130m_stack_static": Workload(
        "m130m_stack_static", SHAPE_130M, batch=8, seqlen=2048, nlayers=24, mode="static",
        calib_seeds=tuple(range(100, 164)), eval_seeds=tuple(range(200, 208)),
        description="24-layer Mamba2-130M-shaped stack, pre-norm residual, batch 8, L 2048, "
                    "static scales calibrated on 64 seeded sequences"),
    "m2p7b_stack": Workload(
        "m2p7b_stack", SHAPE_2P7B, batch=4, seqlen=4096, nlayers=64,
        description="64-layer Mamba2-2.7B-shaped stack, batch 4, L 4096 prefill, dynamic scales"),
    "m2p7b_decode": Workload(
        "m2p7b_decode", SHAPE_2P7B, batch=16, seqlen=1024, nlayers=64, decode_steps=512,
        input_seed=300,
        description="64-layer Mamba2-2.7B-shaped decode, batch 16, 512 one-token steps after "
                    "a 1024-token seeding prefill"),
}

# order of the workloads as listed for the method (small case first)
WORKLOAD_ORDER = ["tiny_layer", "m130m_layer", "m130m_stack_static", "m2p7b_stack", "m2p7b_decode"]


def get(name: str) -> Workload:
    return WORKLOADS[name]


def with_len(w: Workload, batch: int = None, seqlen: int = None) -> Workload:
    """Same workload at another batch / length (parity cases at reduced size)."""
    return replace(w, batch=w.batch if batch is None else batch,
                   seqlen=w.seqlen if seqlen is None else seqlen)
