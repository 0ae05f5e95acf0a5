"""Pins of the layer_norm oracle (CPU only), each against something other than the
oracle's own formula: a hand-worked fixture, torch's layer norm (a separate library
implementation) and its autograd, closed-form moments, invariances, the layout
transpose, and central finite differences of the forward for the gradient."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import layer_norm as oln

HERE = os.path.dirname(os.path.abspath(__file__))


def _fixture():
    with open(os.path.join(HERE, "golden", "layer_norm_hand.json")) as f:
        return json.load(f)


def _val(pairs):
    """[a, c] -> a + c/sqrt(5), elementwise over nested lists."""
    arr = np.asarray(pairs, dtype=np.float64)
    return arr[..., 0] + arr[..., 1] / math.sqrt(5.0)


def test_hand_fixture_forward():
    d = _fixture()
    x = np.asarray(d["x"], np.float32)
    eps = d["epsilon"]
    for key in ("plain", "affine"):
        y, mean, rstd = oln.layer_norm(x, d[key]["g"] if "g" in d[key] else d["affine"]["g"],
                                       d[key]["b"], axis=1, epsilon=eps)
        np.testing.assert_allclose(y, _val(d[key]["y"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(mean, [d["mean"]], atol=1e-15)
        np.testing.assert_allclose(rstd, [_val(d["rstd"])], atol=1e-15)
    y, _, _ = oln.layer_norm(x, d["affine"]["g"], d["affine"]["b"], axis=1, epsilon=eps, relu=True)
    np.testing.assert_allclose(y, _val(d["affine_relu"]["y"]), rtol=0, atol=1e-14)
    # the same vector as a column of a features-first array
    y0, _, _ = oln.layer_norm(x.T.copy(), d["affine"]["g"], d["affine"]["b"], axis=0, epsilon=eps)
    np.testing.assert_allclose(y0.T, _val(d["affine"]["y"]), rtol=0, atol=1e-14)


def test_hand_fixture_grad():
    d = _fixture()
    gr = d["grad"]
    x = np.asarray(d["x"], np.float32)
    dx, dg, db = oln.layer_norm_grad(np.asarray(gr["dy"], np.float32), x, gr["g"], gr["b"], axis=1,
                                     epsilon=d["epsilon"])
    np.testing.assert_allclose(dx, _val(gr["dx"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dg, _val(gr["dg"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(db, _val(gr["db"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("relu", [False, True])
def test_against_torch(relu):
    rng = np.random.default_rng(3)
    N, C = 7, 37
    x = (rng.standard_normal((N, C)) * 3 + 1).astype(np.float32)
    g = rng.standard_normal(C).astype(np.float32)
    b = rng.standard_normal(C).astype(np.float32)
    dy = rng.standard_normal((N, C)).astype(np.float32)
    eps = 1e-6
    y, _, _ = oln.layer_norm(x, g, b, axis=1, epsilon=eps, relu=relu)
    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tg = torch.tensor(g, dtype=torch.float64, requires_grad=True)
    tb = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    ty = torch.nn.functional.layer_norm(tx, (C,), tg, tb, eps)
    if relu:
        ty = torch.relu(ty)
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-12, atol=1e-12)
    ty.backward(torch.tensor(dy, dtype=torch.float64))
    dx, dg, db = oln.layer_norm_grad(dy, x, g, b, axis=1, epsilon=eps, relu=relu)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dg, tg.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(db, tb.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_moments_and_invariance():
    rng = np.random.default_rng(4)
    N, C = 5, 64
    x = (rng.standard_normal((N, C)) * 2 - 3).astype(np.float32)
    ones, zeros = np.ones(C, np.float32), np.zeros(C, np.float32)
    y, mean, rstd = oln.layer_norm(x, ones, zeros, axis=1, epsilon=0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose((y * y).mean(axis=1), 1, atol=1e-12)
    xd = x.astype(np.float64)
    np.testing.assert_allclose(mean, xd.mean(axis=1), atol=1e-13)
    np.testing.assert_allclose(rstd, 1 / xd.std(axis=1), rtol=1e-12)
    # epsilon inside the root: var(y) = var / (var + eps)
    eps = 0.5
    y2, _, _ = oln.layer_norm(x, ones, zeros, axis=1, epsilon=eps)
    var = xd.var(axis=1)
    np.testing.assert_allclose((y2 * y2).mean(axis=1), var / (var + eps), rtol=1e-12)
    # shift and positive scale of the input leave the output unchanged (epsilon = 0)
    x3 = (4 * xd + 7).astype(np.float32)   # rounded to float32: compared to 1e-5
    y3, _, _ = oln.layer_norm(x3, ones, zeros, axis=1, epsilon=0.0)
    np.testing.assert_allclose(y3, y, atol=1e-5)
    # the gain scales and the bias shifts each feature
    g = rng.standard_normal(C).astype(np.float32)
    b = rng.standard_normal(C).astype(np.float32)
    y4, _, _ = oln.layer_norm(x, g, b, axis=1, epsilon=0.0)
    np.testing.assert_allclose(y4, y * g.astype(np.float64) + b.astype(np.float64), atol=1e-13)
    # relu is max(., 0) of the affine output
    y5, _, _ = oln.layer_norm(x, g, b, axis=1, epsilon=0.0, relu=True)
    np.testing.assert_allclose(y5, np.maximum(y4, 0), atol=0)


def test_axis0_is_transpose():
    rng = np.random.default_rng(5)
    C, N = 33, 9
    x = rng.standard_normal((C, N)).astype(np.float32)
    g = rng.standard_normal(C).astype(np.float32)
    b = rng.standard_normal(C).astype(np.float32)
    dy = rng.standard_normal((C, N)).astype(np.float32)
    y0, m0, r0 = oln.layer_norm(x, g, b, axis=0, relu=True)
    y1, m1, r1 = oln.layer_norm(x.T.copy(), g, b, axis=1, relu=True)
    # numpy may sum a transposed view in another order: equal to rounding
    np.testing.assert_allclose(y0, y1.T, rtol=0, atol=1e-13)
    np.testing.assert_allclose(m0, m1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(r0, r1, rtol=1e-13)
    g0 = oln.layer_norm_grad(dy, x, g, b, axis=0, relu=True)
    g1 = oln.layer_norm_grad(dy.T.copy(), x.T.copy(), g, b, axis=1, relu=True)
    np.testing.assert_allclose(g0[0], g1[0].T, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g0[1], g1[1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g0[2], g1[2], rtol=0, atol=1e-12)


@pytest.mark.parametrize("relu", [False, True])
def test_grad_finite_differences(relu):
    """Central differences of the float64 forward; inputs are exact binary fractions so
    the stored float32 values carry no rounding, and no pre-ReLU value sits near 0."""
    rng = np.random.default_rng(6 + relu)
    N, C = 3, 6
    x = (rng.integers(-64, 64, (N, C)) / 16).astype(np.float32)
    g = (rng.integers(-32, 32, C) / 16).astype(np.float32)
    b = (rng.integers(-32, 32, C) / 16).astype(np.float32)
    dy = rng.standard_normal((N, C))
    eps = 1e-3

    def fwd(xd, gd, bd):   # float64 forward on float64 inputs (same definition)
        mean = xd.mean(axis=1, keepdims=True)
        var = ((xd - mean) ** 2).mean(axis=1, keepdims=True)
        y = (xd - mean) / np.sqrt(var + eps) * gd + bd
        return np.maximum(y, 0) if relu else y

    xd, gd, bd = x.astype(np.float64), g.astype(np.float64), b.astype(np.float64)
    m = xd.mean(axis=1, keepdims=True)
    pre = (xd - m) / np.sqrt(((xd - m) ** 2).mean(axis=1, keepdims=True) + eps) * gd + bd
    assert np.abs(pre).min() > 1e-3   # no kink of the ReLU within the difference step
    y, _, _ = oln.layer_norm(x, g, b, axis=1, epsilon=eps, relu=relu)
    np.testing.assert_allclose(y, fwd(x.astype(np.float64), g.astype(np.float64), b.astype(np.float64)),
                               atol=1e-13)
    dx, dg, db = oln.layer_norm_grad(dy.astype(np.float32), x, g, b, axis=1, epsilon=eps, relu=relu)
    dyq = dy.astype(np.float32).astype(np.float64)
    h = 1e-6
    num_dx = np.zeros_like(xd)
    for i in range(N):
        for j in range(C):
            e = np.zeros_like(xd)
            e[i, j] = h
            num_dx[i, j] = ((fwd(xd + e, gd, bd) - fwd(xd - e, gd, bd)) * dyq).sum() / (2 * h)
    num_dg = np.array([((fwd(xd, gd + h * np.eye(C)[j], bd) - fwd(xd, gd - h * np.eye(C)[j], bd)) * dyq).sum() / (2 * h)
                       for j in range(C)])
    num_db = np.array([((fwd(xd, gd, bd + h * np.eye(C)[j]) - fwd(xd, gd, bd - h * np.eye(C)[j])) * dyq).sum() / (2 * h)
                       for j in range(C)])
    np.testing.assert_allclose(dx, num_dx, atol=1e-6)
    np.testing.assert_allclose(dg, num_dg, atol=1e-6)
    np.testing.assert_allclose(db, num_db, atol=1e-6)


def test_decode_exact():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f16 = oln.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    same = (f16 == ref) | (np.isnan(f16) & np.isnan(ref))
    assert same.all()
    bf = oln.decode(bits, "bf16")
    refb = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    sameb = (bf == refb) | (np.isnan(bf) & np.isnan(refb))
    assert sameb.all()
