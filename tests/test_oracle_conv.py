"""The BlocksparseConv oracle against its pins (CPU only): a hand-worked 1-D example
(tests/golden/conv_hand.json) and torch's own dense convolution (conv1d/2d/3d in
float64) of a separately assembled dense filter, with its autograd for the input and
filter gradients, over strides, dilations, SAME / VALID / explicit padding and
overlapping blocks.  None of these calls the oracle to produce an expected value."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import conv as oc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "conv_hand.json")


def test_hand_example():
    h = json.load(open(GOLDEN))
    bck = oc.split_bck(h["bck"])
    I = np.array(h["I"], dtype=np.float64)
    F = np.array(h["F"], dtype=np.float64).reshape(1, 1, 1, 1, 2, 1)
    gv = oc.geometry((2,), (3,), padding="VALID")
    assert np.array_equal(oc.fprop(bck, F, I, h["K"], gv).reshape(1, 2, -1), np.array(h["valid"]["O"]))
    gs = oc.geometry((2,), (3,), strides=(2,), padding="SAME")
    assert gs[2] == (1, 1, 2) and gs[5] == (0, 0, 0)
    assert np.array_equal(oc.fprop(bck, F, I, h["K"], gs).reshape(1, 2, -1), np.array(h["same_stride2"]["O"]))
    dO = np.array(h["updat"]["dO"], dtype=np.float64)
    assert np.array_equal(oc.updat(bck, I, dO, gv).reshape(1, 2), np.array(h["updat"]["dF"]).reshape(1, 2))
    dO = np.array(h["bprop"]["dO"], dtype=np.float64)
    assert np.array_equal(oc.bprop(bck, F, dO, h["C"], gv).reshape(1, 2, 3), np.array(h["bprop"]["dI"]))


def _dense(cl, kl, F, C, K):
    """Dense filter (K, C, T, R, S), each block's taps added at its channel pairs."""
    nb, Bc = cl.shape
    W = np.zeros((K, C) + F.shape[2:5])
    for b in range(nb):
        for i in range(Bc):
            for j in range(kl.shape[1]):
                W[kl[b, j], cl[b, i]] += F[b, i, :, :, :, j]
    return W


def _torch_conv(I5, W, g):
    TRS, DHW, MPQ, st, dl, pads = g
    pad = []
    for a in (2, 1, 0):   # F.pad takes the last dim first
        total = max(0, (MPQ[a] - 1) * st[a] + (TRS[a] - 1) * dl[a] + 1 - DHW[a])
        pad += [pads[a], max(total - pads[a], pads[a])]
    return Fn.conv3d(Fn.pad(I5, pad), W, stride=st, dilation=dl)


CASES = [
    # C, K, Bc, Bk, nblocks, TRS, DHW, strides, dilates, padding
    (6, 5, 2, 3, 4, (3,), (9,), (1,), (1,), "SAME"),
    (8, 8, 4, 4, 3, (3, 3), (7, 6), (2, 1), (1, 1), "SAME"),
    (8, 6, 2, 2, 5, (2, 3), (8, 9), (1, 2), (2, 1), "VALID"),
    (4, 4, 2, 2, 3, (3, 3), (5, 5), (1, 1), (1, 1), 1),
    (6, 6, 3, 3, 2, (2, 3, 2), (4, 5, 6), (1, 2, 1), (1, 1, 2), "SAME"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{len(c[5])}d-{c[9]}" for c in CASES])
def test_against_torch_conv(case):
    C, K, Bc, Bk, nb, TRS, DHW, st, dl, padding = case
    rng = np.random.default_rng(C * 7 + K)
    cl = np.stack([rng.permutation(C)[:Bc] for _ in range(nb)])   # blocks may share channels
    kl = np.stack([rng.permutation(K)[:Bk] for _ in range(nb)])
    g = oc.geometry(TRS, DHW, st, dl, padding)
    N = 3
    F = rng.standard_normal((nb, Bc) + g[0] + (Bk,))
    I = rng.standard_normal((N, C) + tuple(DHW))
    W = _dense(cl, kl, F, C, K)
    It = torch.from_numpy(I.reshape((N, C) + g[1])).requires_grad_()
    Wt = torch.from_numpy(W).requires_grad_()
    Ot = _torch_conv(It, Wt, g)
    assert tuple(Ot.shape[2:]) == g[2]
    O = oc.fprop((cl, kl), F, I, K, g)
    assert np.allclose(O, Ot.detach().numpy(), rtol=1e-12, atol=1e-12)
    dO = rng.standard_normal(Ot.shape)
    Ot.backward(torch.from_numpy(dO))
    assert np.allclose(oc.bprop((cl, kl), F, dO, C, g), It.grad.numpy(), rtol=1e-12, atol=1e-12)
    dW = Wt.grad.numpy()
    dF = oc.updat((cl, kl), I, dO, g)
    for b in range(nb):
        for i in range(Bc):
            for j in range(Bk):
                assert np.allclose(dF[b, i, :, :, :, j], dW[kl[b, j], cl[b, i]], rtol=1e-12, atol=1e-12)


def test_geometry():
    # SAME keeps ceil(X / stride) outputs with the odd pad after; VALID fits whole filters
    assert oc.geometry((3, 3), (7, 8), (2, 2), (1, 1), "SAME")[2:] == ((1, 4, 4), (1, 2, 2), (1, 1, 1), (0, 1, 0))
    assert oc.geometry((3,), (10,), (3,), (2,), "VALID")[2] == (1, 1, 2)
    assert oc.geometry((3,), (10,), (1,), (1,), 2)[2] == (1, 1, 12)
