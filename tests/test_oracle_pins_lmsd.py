"""Pins for the LMSD oracle (HSTU LMSD page, "Overview" equations, dropout off).

Each checks the fp64 oracle against something it does not share code with:
PyTorch's own LayerNorm, SiLU and autograd in fp64, closed forms for constant
rows and u = 0, invariances of the normalisation, and finite differences.  A
dropped affine term, the unbiased variance, a wrong sign in the LayerNorm
backward, a SiLU' slip or a segment read from the wrong offset of dy each fails
at least one of them.
"""

import numpy as np
import pytest
import torch

import oracle
from generative_recommender_attention_amd.workloads import lmsd_named_workload, make_lmsd_workload

F = torch.nn.functional


def torch_lmsd(x, u, w, b, eps, silu_u, concat_u, concat_x):
    d = x.shape[1]
    a = F.silu(u) if silu_u else u
    ln = F.layer_norm(x, (d,), w, b, eps)
    segs = ([a] if concat_u else []) + ([x] if concat_x else []) + [ln * a]
    return torch.cat(segs, dim=1)


FLAGS = [(True, True, True), (True, False, False), (False, True, False), (False, False, True), (True, False, True)]


@pytest.mark.parametrize("flags", FLAGS, ids=[f"silu{int(f[0])}_u{int(f[1])}_x{int(f[2])}" for f in FLAGS])
def test_forward_matches_torch_layer_norm(oracle_lib, flags):
    silu_u, cu, cx = flags
    wl = make_lmsd_workload("pin", 80, 37, 24, silu_u, cu, cx)
    x, u, w, b = (torch.from_numpy(oracle.widen(t)) for t in (wl.x, wl.u, wl.weight, wl.bias))
    want = torch_lmsd(x, u, w, b, wl.eps, silu_u, cu, cx).numpy()
    y, mean, rstd = oracle.lmsd_fwd(wl.x, wl.u, wl.weight, wl.bias, wl.eps, silu_u, cu, cx)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-13)
    var, m = torch.var_mean(x, dim=1, unbiased=False)
    np.testing.assert_allclose(mean, m.numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(rstd, (1.0 / torch.sqrt(var + wl.eps)).numpy(), rtol=1e-13)


@pytest.mark.parametrize("flags", FLAGS, ids=[f"silu{int(f[0])}_u{int(f[1])}_x{int(f[2])}" for f in FLAGS])
def test_backward_matches_torch_autograd(oracle_lib, flags):
    silu_u, cu, cx = flags
    wl = make_lmsd_workload("pin", 81, 29, 40, silu_u, cu, cx)
    x, u, w, b = (torch.from_numpy(oracle.widen(t)).requires_grad_(True) for t in (wl.x, wl.u, wl.weight, wl.bias))
    dy = torch.from_numpy(oracle.widen(wl.dy))
    (torch_lmsd(x, u, w, b, wl.eps, silu_u, cu, cx) * dy).sum().backward()
    _, mean, rstd = oracle.lmsd_fwd(wl.x, wl.u, wl.weight, wl.bias, wl.eps, silu_u, cu, cx)
    dx, du, dw, db = oracle.lmsd_bwd(wl.dy, wl.x, wl.u, wl.weight, wl.bias, mean, rstd, silu_u, cu, cx)
    np.testing.assert_allclose(dx, x.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(du, u.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw, w.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(db, b.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_matches_finite_differences(oracle_lib):
    """Central differences of <dy, y(x, u, weight, bias)> through the oracle's forward."""
    rng = np.random.default_rng(82)
    n, d, eps = 3, 8, 1e-3
    x, u = rng.standard_normal((n, d)), rng.standard_normal((n, d)) * 2.0
    w, b = 1.0 + 0.3 * rng.standard_normal(d), 0.3 * rng.standard_normal(d)
    dy = rng.standard_normal((n, 3 * d))

    def f(xx, uu, ww, bb):
        return float(np.sum(dy * oracle.lmsd_fwd(xx, uu, ww, bb, eps, True, True, True)[0]))

    _, mean, rstd = oracle.lmsd_fwd(x, u, w, b, eps, True, True, True)
    grads = oracle.lmsd_bwd(dy, x, u, w, b, mean, rstd, True, True, True)
    h = 1e-6
    for k, (arr, g) in enumerate(zip((x, u, w, b), grads)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            args_p = [t.copy() for t in (x, u, w, b)]
            args_m = [t.copy() for t in (x, u, w, b)]
            args_p[k][idx] += h
            args_m[k][idx] -= h
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7, err_msg=f"grad {k}")


def test_constant_rows_give_bias_times_activation(oracle_lib):
    """x = c in a row: mean = c, rstd = 1/sqrt(eps), xh = 0, so l = bias and the
    product segment is bias * SiLU(u); the LayerNorm part of dx is 0 (dxh has
    zero mean against xh = 0 only after the mean is removed: dx = rstd (dxh - mean dxh))."""
    rng = np.random.default_rng(83)
    n, d, eps = 4, 16, 1e-2
    x = np.repeat(rng.standard_normal((n, 1)), d, axis=1)
    u, w, b = rng.standard_normal((n, d)), rng.standard_normal(d), rng.standard_normal(d)
    y, mean, rstd = oracle.lmsd_fwd(x, u, w, b, eps, True, False, False)
    np.testing.assert_allclose(mean, x[:, 0], rtol=1e-14)
    np.testing.assert_allclose(rstd, np.full(n, 1.0 / np.sqrt(eps)), rtol=1e-14)
    silu = u / (1.0 + np.exp(-u))
    np.testing.assert_allclose(y, b * silu, rtol=1e-13, atol=1e-15)
    dy = rng.standard_normal((n, d))
    dx, du, dw, db = oracle.lmsd_bwd(dy, x, u, w, b, mean, rstd, True, False, False)
    dxh = dy * silu * w
    np.testing.assert_allclose(dx, (dxh - dxh.mean(axis=1, keepdims=True)) / np.sqrt(eps), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dw, np.zeros(d), atol=1e-13)
    np.testing.assert_allclose(db, (dy * silu).sum(axis=0), rtol=1e-13)


def test_zero_u_closed_form(oracle_lib):
    """u = 0 with SiLU: a = 0, so the product segment and dx's LayerNorm part vanish,
    and du = SiLU'(0) g l = g l / 2."""
    rng = np.random.default_rng(84)
    n, d = 5, 12
    x, u = rng.standard_normal((n, d)), np.zeros((n, d))
    w, b = rng.standard_normal(d), rng.standard_normal(d)
    y, mean, rstd = oracle.lmsd_fwd(x, u, w, b, 1e-6, True, False, True)
    assert np.all(y[:, d:] == 0.0)
    np.testing.assert_array_equal(y[:, :d], x)
    dy = rng.standard_normal((n, 2 * d))
    dx, du, dw, db = oracle.lmsd_bwd(dy, x, u, w, b, mean, rstd, True, False, True)
    np.testing.assert_array_equal(dx, dy[:, :d])     # only the x segment's gradient
    xh = (x - x.mean(axis=1, keepdims=True)) / np.sqrt(x.var(axis=1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(du, 0.5 * dy[:, d:] * (xh * w + b), rtol=1e-12, atol=1e-14)
    assert np.all(dw == 0.0) and np.all(db == 0.0)


def test_normalisation_invariances(oracle_lib):
    """Shifting a row leaves every output of the product segment unchanged; scaling it
    by s with eps scaled by s^2 too."""
    rng = np.random.default_rng(85)
    n, d = 6, 20
    x, u = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    w, b = rng.standard_normal(d), rng.standard_normal(d)
    y0 = oracle.lmsd_fwd(x, u, w, b, 1e-4, True, False, False)[0]
    y1 = oracle.lmsd_fwd(x + 3.25, u, w, b, 1e-4, True, False, False)[0]
    y2 = oracle.lmsd_fwd(x * 4.0, u, w, b, 1e-4 * 16.0, True, False, False)[0]
    np.testing.assert_allclose(y1, y0, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(y2, y0, rtol=1e-12, atol=1e-13)


def test_named_lmsd_workloads_shape():
    wl = lmsd_named_workload("lmsd_n257_d128")
    assert wl.x.shape == (257, 128) and wl.dy.shape == (257, 3 * 128) and wl.segments == 3
    wl = lmsd_named_workload("lmsd_n23460_d512")
    assert wl.n == 23460 and wl.d == 512
