"""Outlier-study baselines against the oracle (bit for bit).

Per-tensor quantization without the rotation, SmoothQuant-style smoothing
factors, the column scaling, and the whole smoothed W8A8 layer through the
library's GEMM, each compared with oracle/outliers.py on seeded inputs with
outlier channels; shapes include a ragged row count and the 130M in_proj.
"""
import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).cuda().contiguous()


def inputs(rows, k, n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k)).astype(np.float32)
    x[:, rng.choice(k, 4, replace=False)] *= 50
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    return x, w


@pytest.mark.parametrize("rows,k,n", [(1, 64, 8), (77, 512, 100), (2048, 768, 3352)])
def test_baselines_match_oracle(rows, k, n):
    from quantized_state_space_fwht_amd import binding as B
    x, w = inputs(rows, k, n, rows + k)
    xd, wd = dev(x), dev(w)
    # per-tensor quantization
    q = torch.empty((rows, k), dtype=torch.int8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    B.fm_quant_per_tensor(xd, q, sc)
    oq, osc = O.outliers.per_tensor_quant(x)
    assert np.array_equal(q.cpu().numpy(), oq) and sc.item() == osc
    # smoothing factors and the scaled operands
    s = torch.empty(k, dtype=torch.float32, device="cuda")
    B.fm_smooth_scales(xd, wd, s)
    os_ = O.outliers.smooth_scales(x, w)
    assert np.array_equal(s.cpu().numpy(), os_)
    xs = torch.empty_like(xd)
    ws = torch.empty_like(wd)
    B.fm_scale_columns(xd, s, True, xs)
    B.fm_scale_columns(wd, s, False, ws)
    assert np.array_equal(xs.cpu().numpy(), (x / os_).astype(np.float32))
    assert np.array_equal(ws.cpu().numpy(), (w * os_).astype(np.float32))
    # the smoothed W8A8 layer end to end
    qa = torch.empty((rows, k), dtype=torch.int8, device="cuda")
    qb = torch.empty((n, k), dtype=torch.int8, device="cuda")
    sa = torch.empty(1, dtype=torch.float32, device="cuda")
    sb = torch.empty(1, dtype=torch.float32, device="cuda")
    B.fm_quant_per_tensor(xs, qa, sa)
    B.fm_quant_per_tensor(ws, qb, sb)
    out = torch.empty((rows, n), dtype=torch.float32, device="cuda")
    B.fm_w8a8_gemm(qa, qb, sa, sb, out=out)
    want = O.outliers.scheme(x, w, "smooth")
    assert np.array_equal(qa.cpu().numpy(), want["a"]) and np.array_equal(qb.cpu().numpy(), want["b"])
    assert np.array_equal(out.cpu().numpy(), want["out"])


def test_zero_tensor_and_zero_columns():
    from quantized_state_space_fwht_amd import binding as B
    x = np.zeros((8, 64), np.float32)
    w = np.ones((4, 64), np.float32)
    w[:, 5] = 0
    q = torch.empty((8, 64), dtype=torch.int8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    B.fm_quant_per_tensor(dev(x), q, sc)
    assert not q.cpu().numpy().any() and sc.item() == 1.0
    x[:, 9] = 3.0
    s = torch.empty(64, dtype=torch.float32, device="cuda")
    B.fm_smooth_scales(dev(x), dev(w), s)
    assert np.array_equal(s.cpu().numpy(), O.outliers.smooth_scales(x, w))
