"""SparseProj host side (CPU only): the feature map the C library builds equals the
oracle's reading for every parameter combination tried (integer work: bit-exact), and
every call validates its arguments before touching the GPU."""
import ctypes

import numpy as np
import pytest

import block_sparse_matrix_amd as bs
from oracle import sparse_proj as sp


@pytest.mark.parametrize("nhidden,nproj,stride,bsz", [
    (64, None, None, 32), (64, 32, None, 32), (64, 32, 32, 16), (100, 24, 9, 8), (8192, 4096, 64, 32),
    (7, 3, None, 1), (33, 32, 1, 1)])
def test_default_map_matches_oracle(nhidden, nproj, stride, bsz):
    p = bs.SparseProj(nhidden, nproj, stride, bsz)
    ref = sp.default_lut(nhidden, nproj, stride, bsz)
    assert p.nhidden == nhidden and p.nproj == ref.size
    assert np.array_equal(p.gather_lut, ref)


def test_given_map_and_rejections():
    rng = np.random.default_rng(0)
    lut = rng.permutation(50)[:17]
    p = bs.SparseProj(50, gather_lut=lut)
    assert np.array_equal(p.gather_lut, lut) and p.nproj == 17
    assert bs.SparseProj(5, gather_lut=[]).nproj == 0
    for bad in ([0, 0], [5], [-1]):
        with pytest.raises(bs.BsmmError):
            bs.SparseProj(5, gather_lut=bad)
    for args in ((8, 6, 4, 2), (8, 4, 1, 2), (8, 3, None, 2), (0, None, None, 1), (8, None, None, 0)):
        with pytest.raises(bs.BsmmError):
            bs.SparseProj(*args)


def test_call_validation_before_gpu():
    L = bs.lib()
    p = bs.SparseProj(64, 32, 32, 16)
    h = p.handle
    vp = ctypes.c_void_p
    good, odd = vp(0x10000), vp(0x10008)
    INVALID, ALIGN = 1, 3
    for fn in (L.bsmm_proj_gather, L.bsmm_proj_scatter):
        assert fn(h, good, good, 4, 2, 0, None) == INVALID       # feature_axis
        assert fn(h, good, good, 4, 1, 7, None) == INVALID       # dtype
        assert fn(h, good, good, -1, 1, 0, None) == INVALID      # N
        assert fn(h, None, good, 4, 1, 0, None) == INVALID
        assert fn(h, good, None, 4, 1, 0, None) == INVALID
        assert fn(h, odd, good, 4, 1, 0, None) == ALIGN
        assert fn(h, None, None, 0, 1, 0, None) == 0             # N = 0: nothing to do
        assert fn(None, good, good, 4, 1, 0, None) == INVALID
    for fn in (L.bsmm_proj_scatter_add, L.bsmm_proj_scatter_mul, L.bsmm_proj_gather_mul):
        assert fn(h, None, good, good, 4, 1, 1, None) == INVALID
        assert fn(h, good, None, good, 4, 1, 1, None) == INVALID
        assert fn(h, good, good, None, 4, 1, 1, None) == INVALID
        assert fn(h, good, good, odd, 4, 0, 2, None) == ALIGN
        assert fn(h, None, None, None, 0, 0, 2, None) == 0
