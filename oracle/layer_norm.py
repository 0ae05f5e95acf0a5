"""CPU oracle for layer_norm -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg import this
module.  The product (block_sparse_matrix_amd and libbsmm.so) never does, and the
two share no code.

Follows the kiteco/blocksparse README, "API Documentation" > blocksparse.norms >
layer_norm(x, g, b, axis=1, epsilon=1e-6, relu=False): a layer norm over the feature
axis of either activation layout of the block-sparse matmul, with an optional ReLU
applied at the end.  The page gives no formula; the plain reading taken here is the
standard one, per normalised vector (a row of x for axis=1, a column for axis=0):

    mean = sum(x) / C,   var = sum((x - mean)^2) / C   (biased),
    xhat = (x - mean) / sqrt(var + epsilon),
    y    = xhat * g + b,  then max(y, 0) when relu,

with g and b per feature (length C, float32 storage).  The gradient is that of this
function: with dyr = dy, or dy * [xhat*g + b > 0] when relu,

    dg = sum over vectors of dyr * xhat,   db = sum over vectors of dyr,
    dx = rstd * (dyr*g - mean(dyr*g) - xhat * mean(dyr*g * xhat)),   rstd = 1/sqrt(var+eps).

Everything is float64 numpy.  Inputs are raw storage: float32 arrays for fp32, uint16
bit patterns for bfloat16 and float16.
"""
from __future__ import annotations

import numpy as np


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements (bf16: the high half of an fp32 word)."""
    a = np.asarray(a)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return a.astype(np.uint16).view(np.float16).astype(np.float64)
    raise ValueError(dtype)


def _rows(x: np.ndarray, axis: int) -> np.ndarray:
    """View with one normalised vector per row."""
    if axis not in (0, 1):
        raise ValueError("axis must be 0 or 1")
    return x if axis == 1 else x.T


def layer_norm(x, g, b, axis: int = 1, epsilon: float = 1e-6, relu: bool = False, dtype: str = "f32"):
    """Forward pass; returns (y, mean, rstd) in float64, y in x's shape."""
    xr = _rows(decode(x, dtype), axis)
    g = np.asarray(g, dtype=np.float32).astype(np.float64)
    b = np.asarray(b, dtype=np.float32).astype(np.float64)
    C = xr.shape[1]
    mean = xr.sum(axis=1) / C
    d = xr - mean[:, None]
    var = (d * d).sum(axis=1) / C
    rstd = 1.0 / np.sqrt(var + epsilon)
    y = d * rstd[:, None] * g[None, :] + b[None, :]
    if relu:
        y = np.maximum(y, 0.0)
    return (y if axis == 1 else y.T), mean, rstd


def layer_norm_grad(dy, x, g, b, axis: int = 1, epsilon: float = 1e-6, relu: bool = False,
                    dtype: str = "f32"):
    """Backward pass; returns (dx, dg, db) in float64 (dx in x's shape)."""
    xr = _rows(decode(x, dtype), axis)
    dyr = _rows(decode(dy, dtype), axis)
    g = np.asarray(g, dtype=np.float32).astype(np.float64)
    b = np.asarray(b, dtype=np.float32).astype(np.float64)
    C = xr.shape[1]
    mean = xr.sum(axis=1) / C
    d = xr - mean[:, None]
    var = (d * d).sum(axis=1) / C
    rstd = 1.0 / np.sqrt(var + epsilon)
    xhat = d * rstd[:, None]
    if relu:
        dyr = dyr * ((xhat * g[None, :] + b[None, :]) > 0)
    dg = (dyr * xhat).sum(axis=0)
    db = dyr.sum(axis=0)
    dxh = dyr * g[None, :]
    dx = rstd[:, None] * (dxh - dxh.mean(axis=1)[:, None] - xhat * (dxh * xhat).mean(axis=1)[:, None])
    return (dx if axis == 1 else dx.T), dg, db
