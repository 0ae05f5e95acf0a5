"""CPU oracle for BlocksparseConv -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg use this module;
the product never imports it and shares no code with it.

The kiteco/blocksparse README ("API Documentation" › blocksparse.conv ›
BlocksparseConv(BCK, TRS, DHW, MPQ=None, strides, dilates, padding, edge_bias)) gives
the constructor and the helpers f_shape / i_shape / o_shape / __call__(F, I), no
formulas.  The readings taken here:

  BCK          blocks; block b lists input channels C_b (Bc of them, distinct) and output
               channels K_b (Bk, distinct); every block has the same Bc and Bk; blocks may
               share channels (their contributions add).
  F            (nblocks, Bc, T, R, S, Bk): F[b, i, t, r, s, j] couples input channel
               C_b[i] at filter tap (t, r, s) to output channel K_b[j].
  I, O         (N, C, D, H, W) and (N, K, M, P, Q) (channels before the spatial dims);
               1-D and 2-D problems are 3-D ones with leading spatial sizes of 1.
  geometry     per spatial dim with size X, filter size F, stride st, dilation dl (an
               integer padding applies to the image's own dims, not the leading 1s):
               "SAME": out = ceil(X / st), pad = max(0, (out-1)*st + (F-1)*dl + 1 - X) // 2
               "VALID": pad = 0, out = (X - (F-1)*dl - 1) // st + 1
               an integer p: pad = p, out = (X + 2p - (F-1)*dl - 1) // st + 1
  fprop        O[n, K_b[j], m, p, q] += sum_{i, t, r, s} I[n, C_b[i], m*st - pad + t*dl, ...]
                                        * F[b, i, t, r, s, j]   over every block b
               (input positions outside the image contribute 0)
  bprop        dI = the gradient of fprop's output with respect to I, given dO
  updat        dF[b, i, t, r, s, j] = sum_{n, m, p, q} I[n, C_b[i], ...] * dO[n, K_b[j], m, p, q]

float64 numpy, one block and one filter tap at a time (einsum over the channel
lists): plain and slow, small inputs only.
"""
from __future__ import annotations

from typing import Sequence, Tuple, Union

import numpy as np


def _dim(X: int, F: int, st: int, dl: int, padding) -> Tuple[int, int]:
    """(output size, leading pad) of one spatial dim."""
    if padding == "SAME":
        out = -(-X // st)
        return out, max(0, (out - 1) * st + (F - 1) * dl + 1 - X) // 2
    if padding == "VALID":
        return (X - (F - 1) * dl - 1) // st + 1, 0
    p = int(padding)
    return (X + 2 * p - (F - 1) * dl - 1) // st + 1, p


def _pad3(v, fill):
    v = tuple(v)
    return (fill,) * (3 - len(v)) + v


def geometry(TRS, DHW, strides=(1, 1, 1), dilates=(1, 1, 1), padding="SAME"):
    """(TRS, DHW, MPQ, strides, dilates, pads) as 3-tuples."""
    nd = len(tuple(DHW))
    TRS, DHW = _pad3(TRS, 1), _pad3(DHW, 1)
    st, dl = _pad3(strides, 1), _pad3(dilates, 1)
    if isinstance(padding, str):
        pads_in = (padding,) * 3
    elif isinstance(padding, (int, np.integer)):
        pads_in = _pad3((int(padding),) * nd, 0)   # the image's own dims only
    else:
        pads_in = _pad3(padding, 0)
    MPQ, pads = [], []
    for a in range(3):
        o, p = _dim(DHW[a], TRS[a], st[a], dl[a], pads_in[a])
        MPQ.append(o)
        pads.append(p)
    return TRS, DHW, tuple(MPQ), st, dl, tuple(pads)


def split_bck(BCK):
    """The pages' BCK (one ((c0, c1, ...), (k0, k1, ...)) pair per block) as two integer
    arrays (nblocks, Bc) and (nblocks, Bk)."""
    cl = np.array([blk[0] for blk in BCK], dtype=np.int64)
    kl = np.array([blk[1] for blk in BCK], dtype=np.int64)
    return cl, kl


def _taps(TRS):
    for t in range(TRS[0]):
        for r in range(TRS[1]):
            for s in range(TRS[2]):
                yield t, r, s


def _window(X: int, out: int, st: int, dl: int, pad: int, tap: int):
    """For output positions 0..out-1: input index out*st - pad + tap*dl, and validity."""
    idx = np.arange(out) * st - pad + tap * dl
    return np.clip(idx, 0, X - 1), (idx >= 0) & (idx < X)


def _shifted(I5: np.ndarray, g, tap) -> np.ndarray:
    """I at the input positions one filter tap reads for every output position
    (zero outside the image): (N, C, M, P, Q)."""
    TRS, DHW, MPQ, st, dl, pads = g
    idx, ok = zip(*[_window(DHW[a], MPQ[a], st[a], dl[a], pads[a], tap[a]) for a in range(3)])
    V = I5[:, :, idx[0]][:, :, :, idx[1]][:, :, :, :, idx[2]]
    mask = ok[0][:, None, None] & ok[1][None, :, None] & ok[2][None, None, :]
    return V * mask


def _as5(a: np.ndarray, spatial) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    return a.reshape(a.shape[:2] + tuple(spatial))


def _as6(F, cl, kl, TRS) -> np.ndarray:
    """The filter as (nblocks, Bc, T, R, S, Bk) (1-D / 2-D filters get leading taps of 1)."""
    return np.asarray(F, dtype=np.float64).reshape((len(cl), len(cl[0])) + tuple(TRS) + (len(kl[0]),))


def fprop(bck, F, I, K: int, g) -> np.ndarray:
    TRS, DHW, MPQ = g[0], g[1], g[2]
    cl, kl = bck
    I5 = _as5(I, DHW)
    F = _as6(F, cl, kl, TRS)
    N = I5.shape[0]
    O = np.zeros((N, K) + MPQ)
    for b in range(len(cl)):
        for tap in _taps(TRS):
            V = _shifted(I5[:, cl[b]], g, tap)             # (N, Bc, M, P, Q)
            O[:, kl[b]] += np.einsum("nimpq,ij->njmpq", V, F[b, :, tap[0], tap[1], tap[2], :])
    return O


def bprop(bck, F, dO, C: int, g) -> np.ndarray:
    """dI: every tap's contribution added back at the input positions it read."""
    TRS, DHW, MPQ, st, dl, pads = g
    cl, kl = bck
    dO5 = _as5(dO, MPQ)
    F = _as6(F, cl, kl, TRS)
    N = dO5.shape[0]
    dI = np.zeros((N, C) + DHW)
    for b in range(len(cl)):
        for tap in _taps(TRS):
            contrib = np.einsum("njmpq,ij->nimpq", dO5[:, kl[b]], F[b, :, tap[0], tap[1], tap[2], :])
            idx, ok = zip(*[_window(DHW[a], MPQ[a], st[a], dl[a], pads[a], tap[a]) for a in range(3)])
            for m in range(MPQ[0]):
                if not ok[0][m]:
                    continue
                for p in range(MPQ[1]):
                    if not ok[1][p]:
                        continue
                    for q in range(MPQ[2]):
                        if ok[2][q]:
                            dI[:, cl[b], idx[0][m], idx[1][p], idx[2][q]] += contrib[:, :, m, p, q]
    return dI


def updat(bck, I, dO, g) -> np.ndarray:
    TRS, DHW, MPQ = g[0], g[1], g[2]
    cl, kl = bck
    I5, dO5 = _as5(I, DHW), _as5(dO, MPQ)
    nb, Bc, Bk = len(cl), len(cl[0]), len(kl[0])
    dF = np.zeros((nb, Bc) + TRS + (Bk,))
    for b in range(nb):
        for tap in _taps(TRS):
            V = _shifted(I5[:, cl[b]], g, tap)
            dF[b, :, tap[0], tap[1], tap[2], :] = np.einsum("nimpq,njmpq->ij", V, dO5[:, kl[b]])
    return dF
