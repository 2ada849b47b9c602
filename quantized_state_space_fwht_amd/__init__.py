"""MI355X-native quantized Mamba2 mixer (FastMamba method).

configs / synth: workload shapes and seeded synthetic inputs (no method arithmetic).
binding:         ctypes marshalling to libfm.so (the HIP kernels behind include/fm.h).
runtime:         device-memory owners (one layer, pre-norm stacks) calling libfm.so.
build:           hipcc build of libfm.so for gfx950.

`binding` and `runtime` import torch and load libfm.so; importing them fails
loudly when the library has not been built.
"""
from . import configs, synth  # noqa: F401

__all__ = ["configs", "synth"]
