"""The oracle's fixed-point scan in plain C (scan_ref.c), for full-size checks.

Test infrastructure, like the rest of oracle/: only tests, the smoke check and
the benchmark's CPU baseline use it.  ``ssm_scan_pot_c`` computes exactly what
scan.ssm_scan_pot computes ([FM] Fig. 2 SSM block; the readings in scan.py),
with the (batch, head) pairs split over threads (ctypes releases the GIL for
the call); the pins check the two against each other and against the closed
forms.  ``build()`` compiles the library with gcc; ``lib()`` builds it when it
is missing.
"""
import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "scan_ref.c")
_LIB = os.path.join(_DIR, "libscan_ref.so")
_lib = None


def build():
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", _SRC, "-o", tmp], check=True)
    os.replace(tmp, _LIB)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_scan_range.restype = i32
        L.oracle_scan_range.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i64, i64, i64, i64, i64,
                                        vp, vp, vp, i64, i64]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def ssm_scan_pot_c(x_q, B_q, C_q, dt, dA, D_q16, p_B, p_C, state_in=None, threads=None):
    """Same arguments and results as scan.ssm_scan_pot (y, state_out int64)."""
    x = np.ascontiguousarray(x_q, dtype=np.int8)
    Bm = np.ascontiguousarray(B_q, dtype=np.int8)
    Cm = np.ascontiguousarray(C_q, dtype=np.int8)
    dt = np.ascontiguousarray(dt, dtype=np.int64)
    dA = np.ascontiguousarray(dA, dtype=np.int64)
    D = np.ascontiguousarray(D_q16, dtype=np.int64)
    Bsz, L, H, P = x.shape
    N = Bm.shape[-1]
    assert Bm.shape == (Bsz, L, N) and Cm.shape == (Bsz, L, N)
    assert dt.shape == (Bsz, L, H) and dA.shape == (Bsz, L, H) and D.shape == (H,)
    st_in = None if state_in is None else np.ascontiguousarray(state_in, dtype=np.int64)
    if st_in is not None:
        assert st_in.shape == (Bsz, H, P, N)
    y = np.zeros((Bsz, L, H, P), dtype=np.int64)
    st = np.zeros((Bsz, H, P, N), dtype=np.int64)
    pairs = Bsz * H
    nt = max(1, min(threads or min(16, os.cpu_count() or 1), pairs))
    bounds = [pairs * i // nt for i in range(nt + 1)]
    f = lib().oracle_scan_range

    def run(i):
        return f(_p(x), _p(Bm), _p(Cm), _p(dt), _p(dA), _p(D), int(p_B), int(p_C), Bsz, L, H, P,
                 N, _p(st_in), _p(y), _p(st), bounds[i], bounds[i + 1])

    with ThreadPoolExecutor(nt) as ex:
        rcs = list(ex.map(run, range(nt)))
    assert all(rc == 0 for rc in rcs), "scan_ref: allocation failed"
    return y, st
