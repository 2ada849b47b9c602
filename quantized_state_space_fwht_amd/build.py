"""Build libfm.so (the HIP kernels + C-ABI) in-tree for gfx950 with hipcc.

    python -m quantized_state_space_fwht_amd.build

Flags: -ffp-contract=off keeps every float32 multiply and add separate (the
rounding of the Hadamard transform, the dequantization and the RMSNorm
decides int8 codes); packed fp32 instructions are disabled.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfm.so")
SOURCES = ["fm_api.hip", "fm_hadamard.hip", "fm_gemm.hip", "fm_conv.hip", "fm_scan.hip",
           "fm_gate.hip", "fm_layer.hip", "fm_nau.hip", "fm_outlier.hip", "fm_state.hip",
           "fm_ssd.hip"]
ARCH = os.environ.get("FM_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           "-I", INCLUDE, "-I", CSRC]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    cmd += ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [l for l in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
