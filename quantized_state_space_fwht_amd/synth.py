"""Seeded synthetic inputs and random-init parameters.

The FastMamba paper evaluates trained Mamba2-130M / 2.7B checkpoints on text
(Section V.A, Table II); neither weights nor datasets are used here.  Instead
every tensor is drawn from numpy's PCG64 generator with a fixed seed:

* activations ~ N(0, 1) with a few fixed channels scaled up (x50), the
  outlier-channel pattern that motivates the Hadamard rotation (Fig. 3,
  activation distributions before the transform; the Mamba-PTQ finding that
  Mamba activations carry outlier channels);
* projection and conv weights ~ N(0, 0.02); dt bias ~ U(-4, -2);
  A = -exp(U(0, 2)); D = 1; gated-RMSNorm weight = 1.

This module only draws numbers.  It holds no step of the method: quantizers,
transforms and fixed-point conversions live on each side (kernels, oracle)
separately.  Both the GPU path and the CPU oracle receive these arrays.
"""
import numpy as np

from .configs import LayerShape, Workload


def outlier_channels(d_model: int, seed: int = 7, count: int = 4) -> np.ndarray:
    """Indices of the outlier channels: first `count` of a seeded permutation, sorted."""
    perm = np.random.default_rng(seed).permutation(d_model)
    return np.sort(perm[:count])


def activations(shape: LayerShape, batch: int, seqlen: int, seed: int,
                outlier_seed: int = 7, n_outliers: int = 4, scale: float = 50.0) -> np.ndarray:
    """u [batch, seqlen, d_model] float32."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((batch, seqlen, shape.d_model), dtype=np.float32)
    idx = outlier_channels(shape.d_model, outlier_seed, n_outliers)
    u[..., idx] *= np.float32(scale)
    return u


def workload_activations(w: Workload, seed: int = None) -> np.ndarray:
    return activations(w.shape, w.batch, w.seqlen, w.input_seed if seed is None else seed,
                       w.outlier_seed, w.n_outliers, w.outlier_scale)


def calibration_sequences(w: Workload):
    """Static mode: one [1, L, d_model] sequence per calibration seed."""
    return [activations(w.shape, 1, w.seqlen, sd, w.outlier_seed, w.n_outliers, w.outlier_scale)
            for sd in w.calib_seeds]


def eval_batch(w: Workload) -> np.ndarray:
    """Static mode: the evaluation sequences (one per seed) as one [B, L, d_model] batch."""
    return np.concatenate([activations(w.shape, 1, w.seqlen, sd, w.outlier_seed, w.n_outliers,
                                       w.outlier_scale) for sd in w.eval_seeds], axis=0)


def decode_step_input(w: Workload, step: int) -> np.ndarray:
    """u_t [batch, d_model] for decode step `step` (seed 400 + step)."""
    return activations(w.shape, w.batch, 1, 400 + step, w.outlier_seed,
                       w.n_outliers, w.outlier_scale)[:, 0, :]


def layer_params(shape: LayerShape, seed: int) -> dict:
    """Random-init float32 parameters of one mixer layer (draw order fixed)."""
    rng = np.random.default_rng(seed)
    s = shape
    p = {}
    p["w_in"] = (rng.standard_normal((s.d_in_proj, s.d_model), dtype=np.float32)
                 * np.float32(0.02))
    p["w_out"] = (rng.standard_normal((s.d_model, s.d_inner), dtype=np.float32)
                  * np.float32(0.02))
    p["conv_w"] = (rng.standard_normal((s.conv_ch, s.d_conv), dtype=np.float32)
                   * np.float32(0.02))
    p["conv_b"] = (rng.standard_normal((s.conv_ch,), dtype=np.float32) * np.float32(0.02))
    p["dt_bias"] = rng.uniform(-4.0, -2.0, size=(s.nheads,)).astype(np.float32)
    p["A"] = (-np.exp(rng.uniform(0.0, 2.0, size=(s.nheads,)))).astype(np.float32)
    p["D"] = np.ones((s.nheads,), dtype=np.float32)
    p["norm_w"] = np.ones((s.d_inner,), dtype=np.float32)
    return p


def workload_params(w: Workload, layer: int) -> dict:
    return layer_params(w.shape, w.param_seed_base + layer)


def nau_knot_tables():
    """Knot tables (nine Q.30 integers, Y_8 = 2 Y_0) for the 8-segment 2^f unit.

    * "chord": Y_i = rint(2^(i/8) * 2^30), the segments' chords.
    * "lsq": the continuous piecewise-linear function on the eighths that
      minimizes the summed squared relative error (P(f) - 2^f) / 2^f over
      the 65536 fractions f = k / 2^16 the unit sees (numpy least squares).
    * "minimax": the same form minimizing the largest relative error over
      those fractions (a linear program, scipy's HiGHS).
    Coefficient inputs of the unit: no step of the layer computes them.
    """
    from scipy.optimize import linprog
    k = np.arange(1 << 16)
    f = k / 65536.0
    seg = k >> 13
    r = (k & 8191) / 8192.0
    a = np.zeros((k.size, 9))
    a[k, seg] = 1.0 - r
    a[k, seg + 1] = r
    a[:, 0] += 2.0 * a[:, 8]          # Y_8 = 2 Y_0: octave continuity
    a = a[:, :8]
    target = 2.0 ** f
    aw = a / target[:, None]          # relative residual (A y - 2^f) / 2^f
    y_lsq = np.linalg.lstsq(aw, np.ones_like(f), rcond=None)[0]
    # minimax: variables (y_0..y_7, t), minimize t with |aw y - 1| <= t
    c = np.zeros(9)
    c[8] = 1.0
    ones = np.ones((k.size, 1))
    a_ub = np.vstack([np.hstack([aw, -ones]), np.hstack([-aw, -ones])])
    b_ub = np.concatenate([np.ones_like(f), -np.ones_like(f)])
    res = linprog(c, A_ub=a_ub, b_ub=b_ub, bounds=[(0.5, 3.0)] * 8 + [(0, None)],
                  method="highs")
    assert res.success, res.message
    y_mm = res.x[:8]

    def q30(y):
        y9 = np.append(y, 2.0 * y[0])
        return np.rint(y9 * 2.0 ** 30).astype(np.int64)

    chord = np.array([int(np.rint(2.0 ** (i / 8.0) * 2.0 ** 30)) for i in range(9)], np.int64)
    return {"chord": chord, "lsq": q30(y_lsq), "minimax": q30(y_mm)}

