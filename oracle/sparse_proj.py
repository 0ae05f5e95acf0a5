"""CPU oracle for SparseProj -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg use this module;
the product never imports it and shares no code with it.

The kiteco/blocksparse README ("API Documentation" › blocksparse.matmul › SparseProj)
gives SparseProj(nhidden, nproj, proj_stride, block_size, gather_lut) with gather,
scatter, scatter_add and scatter_mul: projections between a dense activation of
nhidden features and a sparse one of nproj features through a one-to-one feature map
(no two projected features share a hidden feature, so the backward ops need no
atomics).  The page states no formulas; the readings taken here:

  lut          gather_lut if given (nproj distinct hidden indices); otherwise blocks of
               block_size consecutive hidden features, block j starting at
               j * proj_stride, nproj // block_size blocks (proj_stride defaults to
               block_size, nproj to nhidden).
  gather(x)    y[n, p] = x[n, lut[p]]                                  (N, nproj)
  scatter(x)   y[n, lut[p]] = x[n, p], every other hidden feature 0     (N, nhidden)
  scatter_add  z = x; z[n, lut[p]] = x[n, lut[p]] + y[n, p]             (N, nhidden)
  scatter_mul  z = x; z[n, lut[p]] = x[n, lut[p]] * y[n, p]             (N, nhidden)
  gather_mul   g[n, p] = a[n, lut[p]] * b[n, lut[p]] (the y-gradient of scatter_mul)
The activations are (N, features) for feature_axis 1 and (features, N) for 0.

Values are float64 from exactly decoded inputs; floating-point results (add, mul) are
the exact fp64 operations, which the tests compare to the device within tolerance.
Pure numpy indexing and loops: plain and slow, small inputs only.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def default_lut(nhidden: int, nproj: Optional[int] = None, proj_stride: Optional[int] = None,
                block_size: int = 32) -> np.ndarray:
    """The feature map when no gather_lut is given: nproj // block_size blocks of
    block_size consecutive hidden features, block j starting at j * proj_stride."""
    nproj = nhidden if nproj is None else nproj
    stride = block_size if proj_stride is None else proj_stride
    if nproj % block_size or stride < block_size:
        raise ValueError("nproj must be whole blocks and proj_stride >= block_size")
    lut = []
    for j in range(nproj // block_size):
        for i in range(block_size):
            lut.append(j * stride + i)
    lut = np.array(lut, dtype=np.int64)
    if lut.size and lut.max() >= nhidden:
        raise ValueError("the blocks run past nhidden")
    return lut


def check_lut(lut: Sequence[int], nhidden: int) -> np.ndarray:
    """A one-to-one map of projected features into [0, nhidden)."""
    a = np.asarray(lut, dtype=np.int64)
    if a.ndim != 1 or (a.size and (a.min() < 0 or a.max() >= nhidden)) or np.unique(a).size != a.size:
        raise ValueError("gather_lut must hold distinct indices in [0, nhidden)")
    return a


def _feat_last(a: np.ndarray, fa: int) -> np.ndarray:
    return np.asarray(a, dtype=np.float64) if fa == 1 else np.asarray(a, dtype=np.float64).T


def _back(a: np.ndarray, fa: int) -> np.ndarray:
    return a if fa == 1 else np.ascontiguousarray(a.T)


def gather(lut, x, fa: int = 1) -> np.ndarray:
    xf = _feat_last(x, fa)
    y = np.empty((xf.shape[0], len(lut)))
    for p, h in enumerate(lut):
        y[:, p] = xf[:, h]
    return _back(y, fa)


def scatter(lut, x, nhidden: int, fa: int = 1) -> np.ndarray:
    xf = _feat_last(x, fa)
    y = np.zeros((xf.shape[0], nhidden))
    for p, h in enumerate(lut):
        y[:, h] = xf[:, p]
    return _back(y, fa)


def scatter_add(lut, x, y, fa: int = 1) -> np.ndarray:
    z = _feat_last(x, fa).copy()
    yf = _feat_last(y, fa)
    for p, h in enumerate(lut):
        z[:, h] = z[:, h] + yf[:, p]
    return _back(z, fa)


def scatter_mul(lut, x, y, fa: int = 1) -> np.ndarray:
    z = _feat_last(x, fa).copy()
    yf = _feat_last(y, fa)
    for p, h in enumerate(lut):
        z[:, h] = z[:, h] * yf[:, p]
    return _back(z, fa)


def gather_mul(lut, a, b, fa: int = 1) -> np.ndarray:
    af, bf = _feat_last(a, fa), _feat_last(b, fa)
    g = np.empty((af.shape[0], len(lut)))
    for p, h in enumerate(lut):
        g[:, p] = af[:, h] * bf[:, h]
    return _back(g, fa)
