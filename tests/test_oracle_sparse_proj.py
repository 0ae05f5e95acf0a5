"""The SparseProj oracle against its pins (CPU only): a hand-worked example
(tests/golden/sparse_proj_hand.json), torch's own indexing routines, and the identities
a one-to-one feature map fixes (gather after scatter is the identity, scatter after
gather masks, adjointness of gather and scatter, scatter_add = x + scatter, scatter_mul
by ones is the identity, the feature-axis transpose).  None of these calls the oracle to
produce an expected value."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import sparse_proj as sp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sparse_proj_hand.json")


def test_hand_example():
    g = json.load(open(GOLDEN))
    lut = sp.check_lut(g["lut"], g["nhidden"])
    x = np.array(g["x"], dtype=np.float64)
    s = np.array(g["s"], dtype=np.float64)
    assert np.array_equal(sp.gather(lut, x), np.array(g["gather_x"]))
    assert np.array_equal(sp.scatter(lut, s, g["nhidden"]), np.array(g["scatter_s"]))
    assert np.array_equal(sp.scatter_add(lut, x, s), np.array(g["scatter_add"]))
    assert np.array_equal(sp.scatter_mul(lut, x, s), np.array(g["scatter_mul"]))
    assert np.array_equal(sp.gather_mul(lut, x, x), np.array(g["gather_mul_xx"]))
    for case in g["default_luts"]:
        got = sp.default_lut(case["nhidden"], case["nproj"], case["proj_stride"], case["block_size"])
        assert got.tolist() == case["lut"]


def _case(seed, H=40, P=13, N=7):
    rng = np.random.default_rng(seed)
    lut = rng.permutation(H)[:P]
    x = rng.standard_normal((N, H))
    s = rng.standard_normal((N, P))
    return lut, x, s


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_against_torch_indexing(seed):
    lut, x, s = _case(seed)
    H = x.shape[1]
    tl = torch.from_numpy(lut)
    tx, ts = torch.from_numpy(x), torch.from_numpy(s)
    assert np.array_equal(sp.gather(lut, x), torch.index_select(tx, 1, tl).numpy())
    assert np.array_equal(sp.scatter(lut, s, H), torch.zeros(x.shape, dtype=torch.float64).index_copy(1, tl, ts).numpy())
    assert np.array_equal(sp.scatter_add(lut, x, s), tx.index_add(1, tl, ts).numpy())
    ref_mul = tx.clone()
    ref_mul[:, tl] = tx[:, tl] * ts
    assert np.array_equal(sp.scatter_mul(lut, x, s), ref_mul.numpy())


@pytest.mark.parametrize("seed", [3, 4])
def test_identities(seed):
    lut, x, s = _case(seed)
    H = x.shape[1]
    mask = np.zeros(H)
    mask[lut] = 1
    assert np.array_equal(sp.gather(lut, sp.scatter(lut, s, H)), s)
    assert np.array_equal(sp.scatter(lut, sp.gather(lut, x), H), x * mask)
    # adjoint: <gather(x), s> = <x, scatter(s)>
    assert abs(np.sum(sp.gather(lut, x) * s) - np.sum(x * sp.scatter(lut, s, H))) < 1e-12
    assert np.array_equal(sp.scatter_add(lut, x, s), x + sp.scatter(lut, s, H))
    assert np.array_equal(sp.scatter_mul(lut, x, np.ones_like(s)), x)
    assert np.array_equal(sp.scatter_mul(lut, x, s), x * (sp.scatter(lut, s, H) + (1 - mask)))
    assert np.array_equal(sp.gather_mul(lut, x, 2 * x), sp.gather(lut, x) * sp.gather(lut, 2 * x))
    # feature_axis 0 is the same map on transposed activations
    for f, args in ((sp.gather, (x,)), (sp.scatter_add, (x, s)), (sp.scatter_mul, (x, s))):
        assert np.array_equal(f(lut, *[a.T for a in args], fa=0), f(lut, *args).T)
    assert np.array_equal(sp.scatter(lut, s.T, H, fa=0), sp.scatter(lut, s, H).T)


def test_lut_checks():
    with pytest.raises(ValueError):
        sp.check_lut([0, 0], 4)
    with pytest.raises(ValueError):
        sp.check_lut([4], 4)
    with pytest.raises(ValueError):
        sp.default_lut(8, 4, 1, 2)      # overlapping blocks
    with pytest.raises(ValueError):
        sp.default_lut(8, 6, 4, 2)      # third block starts at 8
    assert sp.default_lut(64, 32, 32, 16).tolist() == list(range(16)) + list(range(32, 48))
