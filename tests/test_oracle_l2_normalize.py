"""Pins of the l2_normalize oracle (CPU only): a hand-worked fixture, torch's weight
normalisation of the masked dense weight (a separate implementation) and its autograd,
column norms equal to |gain|, the epsilon branch of an all-zero column, and central
finite differences for the gradient."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import l2_normalize as ol2

HERE = os.path.dirname(os.path.abspath(__file__))


def _dense(layout, blocks, b):
    """Masked dense C x K weight from the stored blocks (row-major block ids)."""
    L = np.asarray(layout)
    R, S = L.shape
    out = np.zeros((R * b, S * b))
    bid = 0
    for c in range(R):
        for k in range(S):
            if L[c, k]:
                out[c * b:(c + 1) * b, k * b:(k + 1) * b] = blocks[bid]
                bid += 1
    return out


def _blocks(layout, dense, b):
    L = np.asarray(layout)
    return np.stack([dense[c * b:(c + 1) * b, k * b:(k + 1) * b] for c, k in zip(*np.nonzero(L))])


def test_hand_fixture():
    with open(os.path.join(HERE, "golden", "l2_normalize_hand.json")) as f:
        d = json.load(f)
    w = np.asarray(d["w"], np.float32)
    out, n = ol2.l2_normalize(d["layout"], w, d["block_size"], d["gain"], epsilon=1e-6)
    np.testing.assert_allclose(n, d["norm"], atol=1e-15)
    np.testing.assert_allclose(out, d["out"], atol=1e-15)
    dw, dg = ol2.l2_normalize_grad(d["layout"], np.asarray(d["dy"], np.float32), w, d["block_size"], d["gain"])
    np.testing.assert_allclose(dw, d["dw"], atol=1e-15)
    np.testing.assert_allclose(dg, d["dgain"], atol=1e-15)


@pytest.mark.parametrize("b,with_gain", [(8, True), (16, False), (32, True)])
def test_against_torch_weight_norm(b, with_gain):
    rng = np.random.default_rng(b)
    L = (rng.random((5, 4)) < 0.5).astype(np.uint8)
    L[:, 0] = 1
    nnz = int(L.sum())
    w = rng.standard_normal((nnz, b, b)).astype(np.float32)
    g = rng.standard_normal(4 * b).astype(np.float32) if with_gain else None
    dy = rng.standard_normal((nnz, b, b)).astype(np.float32)
    out, n = ol2.l2_normalize(L, w, b, g)
    V = torch.tensor(_dense(L, w.astype(np.float64), b), requires_grad=True)
    G = torch.tensor(np.ones(4 * b) if g is None else g.astype(np.float64), requires_grad=True)
    Wn = torch._weight_norm(V, G.view(1, -1), 1)   # norm over dim 0 (inputs), per output column
    np.testing.assert_allclose(out, _blocks(L, Wn.detach().numpy(), b), rtol=1e-12, atol=1e-12)
    (Wn * torch.tensor(_dense(L, dy.astype(np.float64), b))).sum().backward()
    dw, dg = ol2.l2_normalize_grad(L, dy, w, b, g)
    np.testing.assert_allclose(dw, _blocks(L, V.grad.numpy(), b), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dg, G.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_column_norms_equal_gain():
    rng = np.random.default_rng(3)
    L = (rng.random((6, 6)) < 0.4).astype(np.uint8)
    L[np.arange(6), np.arange(6)] = 1
    b = 8
    w = rng.standard_normal((int(L.sum()), b, b)).astype(np.float32)
    g = (rng.random(6 * b) + 0.5).astype(np.float32)
    out, _ = ol2.l2_normalize(L, w, b, g)
    cols = np.sqrt((_dense(L, out, b) ** 2).sum(axis=0))
    np.testing.assert_allclose(cols, g.astype(np.float64), rtol=1e-12)


def test_zero_column_epsilon_branch():
    """An all-zero column: n = sqrt(epsilon), the output stays 0, dW = g/sqrt(eps) * dy, dg = 0."""
    L = np.array([[1, 1]], np.uint8)
    b, eps = 2, 1e-6
    w = np.zeros((2, b, b), np.float32)
    w[0] = [[1, 2], [3, 4]]   # block column 0 nonzero; block column 1 all zero
    dy = np.ones((2, b, b), np.float32)
    g = np.array([1, 1, 2, 2], np.float32)
    out, n = ol2.l2_normalize(L, w, b, g, eps)
    assert np.all(out[1] == 0) and np.allclose(n[2:], np.sqrt(eps))
    dw, dg = ol2.l2_normalize_grad(L, dy, w, b, g, eps)
    np.testing.assert_allclose(dw[1], 2 / np.sqrt(eps) * dy[1], rtol=1e-12)
    np.testing.assert_allclose(dg[2:], 0, atol=0)


def test_grad_finite_differences():
    rng = np.random.default_rng(9)
    L = np.array([[1, 0], [1, 1]], np.uint8)
    b = 2
    w = (rng.integers(-8, 9, (3, b, b)) / 4).astype(np.float32)
    w[:, 0, :] += 3   # keep every column's sum of squares well above epsilon
    g = np.array([1.5, -0.5, 2.0, 0.25], np.float32)
    dy = rng.standard_normal((3, b, b))
    dyq = dy.astype(np.float32).astype(np.float64)

    def f(wd, gd):
        out = np.empty_like(wd)
        cs, ks = np.nonzero(L)   # row-major block ids
        sq = np.zeros(2 * b)
        for bid, k in enumerate(ks):
            sq[k * b:(k + 1) * b] += (wd[bid] ** 2).sum(axis=0)
        nn = np.sqrt(sq)
        for bid, k in enumerate(ks):
            out[bid] = wd[bid] * (gd[k * b:(k + 1) * b] / nn[k * b:(k + 1) * b])[None, :]
        return (out * dyq).sum()

    wd, gd = w.astype(np.float64), g.astype(np.float64)
    h = 1e-6
    num_w = np.zeros_like(wd)
    for idx in np.ndindex(wd.shape):
        e = np.zeros_like(wd)
        e[idx] = h
        num_w[idx] = (f(wd + e, gd) - f(wd - e, gd)) / (2 * h)
    num_g = np.array([(f(wd, gd + h * np.eye(2 * b)[j]) - f(wd, gd - h * np.eye(2 * b)[j])) / (2 * h)
                      for j in range(2 * b)])
    dw, dg = ol2.l2_normalize_grad(L, dy.astype(np.float32), w, b, g)
    np.testing.assert_allclose(dw, num_w, atol=1e-6)
    np.testing.assert_allclose(dg, num_g, atol=1e-6)
