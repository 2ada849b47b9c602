"""Pin strength: plausible mistakes planted in a copy of the oracle fail a pin.

Each case copies the repository's sources to a temporary directory, replaces
one line of the oracle with a plausible mistake (a dropped rounding term, a
wrong shift, sign, index, operand or byte order, a parameter ignored), and
runs the oracle pins there in a subprocess; the case passes when that run
reports a failed pin.  A control runs the same pins on an unmodified copy.
CPU only; the planted mistakes never leave the temporary copy.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (file, original text, planted mistake)
MUTATIONS = [
    ("oracle/layer.py", "xbc = v[:, di:di + ch]",
     "xbc = np.concatenate([v[:, di + di:di + ch], v[:, di:di + di]], axis=1)"),
    ("oracle/hadamard.py", "v = np.stack((a + b, a - b), axis=2)",
     "v = np.stack((a + b, b - a), axis=2)"),
    ("oracle/scan.py", "num = dA[:, t, :, None, None] * h + inc + (1 << 15)",
     "num = dA[:, t, :, None, None] * h + inc"),
    ("oracle/scan.py", "inc = (u[..., None] * Bm[:, t, None, None, :]) << 8",
     "inc = (u[..., None] * Bm[:, t, None, None, :]) << 7"),
    ("oracle/layer.py", "p_y = p_x + 8", "p_y = p_x + 7"),
    ("oracle/scan.py", "y[:, t] = sat32(rshr(y_acc, ky) + rshr(D[None, :, None] * x[:, t], 8))",
     "y[:, t] = sat32(rshr(y_acc, ky))"),
    ("oracle/nau.py", "sig = (e << 16) // ((1 << 16) + e)", "sig = (e << 16) // ((1 << 16) + 2 * e)"),
    ("oracle/nau.py", "i = f >> 13", "i = f >> 14"),
    ("oracle/gate_norm.py", "ms = ss / np.float32(D)", "ms = ss / np.float32(D - 1)"),
    ("oracle/conv.py", "shift = int(p_c) + np.asarray(p_w, dtype=np.int64) - 16",
     "shift = int(p_c) + np.asarray(p_w, dtype=np.int64) - 15"),
    ("oracle/conv.py", "acc += w[None, None, :, k] * padded[:, k:k + L, :]",
     "acc += w[None, None, :, 3 - k] * padded[:, k:k + L, :]"),
    ("oracle/scan.py", "arg = sat32(rshr(dt * np.asarray(A_q16, dtype=np.int64), 16))",
     "arg = sat32(rshr(dt * np.asarray(A_q16, dtype=np.int64), 17))"),
    ("oracle/linear.py",
     "acc = (a.astype(np.float64) @ b.astype(np.float64).T).astype(np.int64)",
     "acc = (a.astype(np.float64) @ b.astype(np.float64)[::-1].T).astype(np.int64)"),
    ("oracle/layer.py", "dt_raw = v[:, di + ch:di + ch + H]", "dt_raw = v[:, di + ch - H:di + ch]"),
    ("oracle/gate_norm.py", "return y_f * sz", "return y_f * np.float32(z)"),
    # narrow state caches
    ("oracle/scan.py", "c = (h + ((1 << shift) >> 1)) >> shift", "c = h >> shift"),
    ("oracle/scan.py", "lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1",
     "lo, hi = -(1 << (bits - 1)), (1 << bits) - 1"),
    ("oracle/scan.py", "out[:, k] = (u >> (8 * k)) & 0xFF", "out[:, nb - 1 - k] = (u >> (8 * k)) & 0xFF"),
    # the recurrence without rounding (chunked variant)
    ("oracle/scan.py", "u = dtf[:, t, :, None] * x[:, t] / 256.0", "u = dtf[:, t, :, None] * x[:, t] / 128.0"),
    ("oracle/scan.py", "h = a[:, t, :, None, None] * h + u[..., None] * Bm[:, t, None, None, :]",
     "h = h + u[..., None] * Bm[:, t, None, None, :]"),
    # the C twin of the scan
    ("oracle/scan_ref.c", "const int64_t num = dav * hr[n] + inc + ((int64_t)1 << 15);",
     "const int64_t num = dav * hr[n] + inc;"),
    # fitted knot tables, quantization statistics, smoothing
    ("oracle/nau.py", "tab = EXP2_TABLE_Q30 if table is None else np.asarray(table, dtype=np.int64)",
     "tab = EXP2_TABLE_Q30"),
    ("oracle/quant_stats.py", "return _summary(r, q, step, np.abs(rc) > 127)",
     "return _summary(r, q, step, np.abs(rc) > 128)"),
    ("oracle/outliers.py", "s[ok] = (np.sqrt(ax[ok]) / np.sqrt(aw[ok])).astype(np.float32)",
     "s[ok] = (np.sqrt(aw[ok]) / np.sqrt(ax[ok])).astype(np.float32)"),
    # calibration: the running maximum replaced by the last sequence's, or one sequence only
    ("oracle/layer.py", "self.amax_u = max(self.amax_u, other.amax_u)", "self.amax_u = other.amax_u"),
    ("oracle/layer.py", "self.amax_q16 = [max(a, b) for a, b in zip(self.amax_q16, other.amax_q16)]",
     "self.amax_q16 = list(other.amax_q16)"),
    ("oracle/layer.py", "    for u in calib_inputs:", "    for u in calib_inputs[:1]:"),
    # stack decode: the pre-norm dropped, or the residual dropped
    ("oracle/layer.py", "        xin = rmsnorm_fixed_order(h, ones)", "        xin = h"),
    ("oracle/layer.py", "        h = h + out\n        new_caches.append(cache)",
     "        h = out\n        new_caches.append(cache)"),
]


def _copy(dst):
    """The pins need the oracle, the tests and the package's configs / synth."""
    skip = shutil.ignore_patterns("__pycache__", ".pytest_cache", "*.so", "csrc")
    for sub in ("oracle", "tests", "quantized_state_space_fwht_amd"):
        shutil.copytree(os.path.join(ROOT, sub), os.path.join(dst, sub), ignore=skip)


def _run_pins(root):
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           "-m", "not gpu", "tests/test_oracle_pins.py"],
                          cwd=root, capture_output=True, text=True, timeout=600)


def test_unmodified_copy_passes_the_pins(tmp_path):
    root = str(tmp_path / "repo")
    _copy(root)
    r = _run_pins(root)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("path,old,new", MUTATIONS,
                         ids=[f"{i:02d}-{os.path.basename(m[0])}" for i, m in enumerate(MUTATIONS)])
def test_planted_mistake_fails_a_pin(tmp_path, path, old, new):
    root = str(tmp_path / "repo")
    _copy(root)
    f = os.path.join(root, path)
    src = open(f).read()
    assert src.count(old) == 1, f"{path}: the original text is not there exactly once"
    open(f, "w").write(src.replace(old, new))
    r = _run_pins(root)
    assert r.returncode == 1 and " failed" in r.stdout, \
        f"planted mistake not caught ({path}: {new})\n" + r.stdout[-1500:]
