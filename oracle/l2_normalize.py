"""CPU oracle for BlocksparseMatMul.l2_normalize -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg import this
module.  The product (block_sparse_matrix_amd and libbsmm.so) never does, and the
two share no code.

Follows the kiteco/blocksparse README, "API Documentation" > blocksparse.matmul >
BlocksparseMatMul.l2_normalize(W, gain=None, epsilon=1e-6, dtype=np.float32): weight
normalisation of the stored blocks.  The page gives only the signature; the plain
reading taken here is weight normalisation per output feature of y = x . W~ (a column
of the masked dense W~), with the l2_normalize convention for epsilon:

    n[o]  = sqrt(max(sum over the column's stored weights of W^2, epsilon)),
            o = k*b + j, the sum over every block (c, k) present and every row i,
    out   = W[id(c,k)][i][j] * g[o] / n[o]      (g = 1 when no gain is given),

and its gradient for an upstream dOut (same layout):

    s[o]  = sum over the column of dOut * W,
    dW    = g[o]/n[o] * (dOut - W * s[o] / n[o]^2)   if the column's sum of squares > epsilon,
            g[o]/n[o] * dOut                         otherwise (n is then the constant sqrt(epsilon)),
    dg[o] = s[o] / n[o].

Block ids number the layout's nonzeros row-major (the matmul's convention).  Inputs are
raw storage (float32, or uint16 bit patterns for bfloat16/float16); outputs float64.
"""
from __future__ import annotations

import numpy as np

from .layer_norm import decode


def _ids(layout):
    L = np.asarray(layout)
    cs, ks = np.nonzero(L)   # row-major order = block id order
    return cs, ks, L.shape[1]


def column_norms(layout, w, block: int, epsilon: float = 1e-6, dtype: str = "f32"):
    """(n, sumsq): per output feature, length K = S * block."""
    cs, ks, S = _ids(layout)
    W = decode(w, dtype).reshape(len(cs), block, block)
    sumsq = np.zeros(S * block)
    for bid in range(len(cs)):
        k = ks[bid]
        sumsq[k * block:(k + 1) * block] += (W[bid] ** 2).sum(axis=0)   # over rows i, per column j
    return np.sqrt(np.maximum(sumsq, epsilon)), sumsq


def l2_normalize(layout, w, block: int, gain=None, epsilon: float = 1e-6, dtype: str = "f32"):
    cs, ks, S = _ids(layout)
    W = decode(w, dtype).reshape(len(cs), block, block)
    n, _ = column_norms(layout, w, block, epsilon, dtype)
    g = np.ones(S * block) if gain is None else np.asarray(gain, np.float32).astype(np.float64)
    out = np.empty_like(W)
    for bid in range(len(cs)):
        k = ks[bid]
        sl = slice(k * block, (k + 1) * block)
        out[bid] = W[bid] * (g[sl] / n[sl])[None, :]
    return out, n


def l2_normalize_grad(layout, dy, w, block: int, gain=None, epsilon: float = 1e-6, dtype: str = "f32",
                      dy_dtype: str = "f32"):
    cs, ks, S = _ids(layout)
    W = decode(w, dtype).reshape(len(cs), block, block)
    D = decode(dy, dy_dtype).reshape(len(cs), block, block)
    n, sumsq = column_norms(layout, w, block, epsilon, dtype)
    g = np.ones(S * block) if gain is None else np.asarray(gain, np.float32).astype(np.float64)
    s = np.zeros(S * block)
    for bid in range(len(cs)):
        k = ks[bid]
        s[k * block:(k + 1) * block] += (D[bid] * W[bid]).sum(axis=0)
    active = sumsq > epsilon
    dW = np.empty_like(W)
    for bid in range(len(cs)):
        k = ks[bid]
        sl = slice(k * block, (k + 1) * block)
        corr = np.where(active[sl], s[sl] / n[sl] ** 2, 0.0)
        dW[bid] = (g[sl] / n[sl])[None, :] * (D[bid] - W[bid] * corr[None, :])
    dg = s / n
    return dW, dg
