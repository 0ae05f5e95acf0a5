"""BlocksparseConv host side (CPU only): the output size and pads the C library
computes equal the oracle's reading for every geometry tried, bad plans are rejected,
and calls validate their arguments before touching the GPU."""
import ctypes

import numpy as np
import pytest

import block_sparse_matrix_amd as bs
from oracle import conv as oc

BCK = (((0, 1), (2, 3)), ((2, 3), (0, 1)))


@pytest.mark.parametrize("TRS,DHW,st,dl,pad", [
    ((3,), (9,), (1,), (1,), "SAME"), ((3, 3), (7, 8), (2, 2), (1, 1), "SAME"), ((2, 3), (8, 9), (1, 2), (2, 1), "VALID"),
    ((3, 3), (5, 5), (1, 1), (1, 1), 1), ((2, 3, 2), (4, 5, 6), (1, 2, 1), (1, 1, 2), "SAME"),
    ((5,), (11,), (3,), (2,), "SAME"), ((1, 1), (4, 4), (2, 2), (1, 1), "VALID"), ((3, 3), (6, 7), (1, 1), (2, 2), (2, 1))])
def test_geometry_matches_oracle(TRS, DHW, st, dl, pad):
    c = bs.BlocksparseConv(BCK, TRS, DHW, strides=st, dilates=dl, padding=pad)
    g = oc.geometry(TRS, DHW, st, dl, pad)
    nd = len(DHW)
    assert c.MPQ == g[2][3 - nd:] and c.pads == g[5][3 - nd:]
    assert c.f_shape() == (2, 2) + tuple(TRS) + (2,) and c.i_shape(5) == (5, 4) + tuple(DHW)


def test_rejections():
    for bck in ((((0, 0), (1, 2)),), (((0, 1), (1, 1)),), (((0, 1), tuple(range(65))),)):
        with pytest.raises(bs.BsmmError):
            bs.BlocksparseConv(bck, (3,), (9,))
    with pytest.raises(bs.BsmmError):
        bs.BlocksparseConv(BCK, (5,), (3,), padding="VALID")   # the filter does not fit
    with pytest.raises(NotImplementedError):
        bs.BlocksparseConv(BCK, (3,), (9,), edge_bias=True)
    with pytest.raises(ValueError):
        bs.BlocksparseConv(BCK, (3,), (9,), MPQ=(4,))


def test_call_validation_before_gpu():
    L = bs.lib()
    c = bs.BlocksparseConv(BCK, (3, 3), (8, 8))
    h = c.handle
    vp = ctypes.c_void_p
    good, odd = vp(0x10000), vp(0x10008)
    INVALID, ALIGN = 1, 3
    upd = lambda *a: L.bsmm_conv_updat(*a[:-1], None, 0, a[-1])   # no workspace
    for fn in (L.bsmm_conv_fprop, L.bsmm_conv_bprop, upd):
        assert fn(h, good, good, good, 2, 7, None) == INVALID
        assert fn(h, good, good, good, -1, 0, None) == INVALID
        assert fn(h, good, good, None, 2, 0, None) == INVALID
        assert fn(h, None, good, good, 2, 0, None) == INVALID
        assert fn(h, good, None, good, 2, 0, None) == INVALID
        assert fn(h, good, odd, good, 2, 1, None) == ALIGN
        assert fn(None, good, good, good, 2, 0, None) == INVALID
    n = ctypes.c_size_t(7)
    assert L.bsmm_conv_workspace_size(h, 64, 1, ctypes.byref(n)) == 0 and n.value == 0   # 2-channel blocks: direct
    c16 = bs.BlocksparseConv([(tuple(range(16)), tuple(range(16)))], (3, 3), (8, 8))
    # fp32: the gathering filter gradient, 16 parts (64 images of one 128-position step, at
    # least 4 steps per part) of 16 x 9 x 16 fp32 partials
    assert L.bsmm_conv_workspace_size(c16.handle, 64, 0, ctypes.byref(n)) == 0 and n.value == 16 * 16 * 9 * 16 * 4
    assert L.bsmm_conv_workspace_size(c16.handle, 8, 0, ctypes.byref(n)) == 0 and n.value == 2 * 16 * 9 * 16 * 4
    assert L.bsmm_conv_workspace_size(c16.handle, 64, 1, ctypes.byref(n)) == 0
    assert n.value == 16 * 16 * 16 * 9 * 4                      # 16 parts of 16 x 9 x 16 fp32 partials
    assert L.bsmm_conv_fprop(h, None, None, None, 0, 0, None) == 0
    assert L.bsmm_conv_bprop(h, None, None, None, 0, 0, None) == 0


def test_plan_without_blocks_takes_the_direct_kernels():
    """A plan with no block (C API only) writes zero outputs through the direct kernels."""
    L = bs.lib()
    h = ctypes.c_void_p()
    a3 = lambda *v: (ctypes.c_int64 * 3)(*v)
    assert L.bsmm_conv_create(ctypes.byref(h), 0, 32, 32, None, None, 64, 64, a3(1, 3, 3), a3(1, 8, 8),
                              a3(1, 1, 1), a3(1, 1, 1), 0, None) == 0
    name = ctypes.c_char_p()
    for p in (0, 1, 2):
        assert L.bsmm_conv_kernel_name(h, p, 1, ctypes.byref(name)) == 0
        assert name.value == (b"direct" if p < 2 else b"matrix_core")
    L.bsmm_conv_destroy(h)
