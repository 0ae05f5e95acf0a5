"""Seeded synthetic inputs for the block-sparse matmul (layouts, weights, activations).

This module only draws random numbers and block layouts.  It holds none of the
arithmetic of the method: no products, sums or reductions of the operands.  Both
the CPU oracle (through the tests) and the HIP path consume what it produces.

The workloads follow the kiteco/blocksparse README, section "Usage": a square
hidden size, a block size from {8, 16, 32} ("API Documentation" ›
blocksparse.matmul › BlocksparseMatMul.__init__), a random 0/1 block layout and a
minibatch of activations.  Six named workloads are defined (WORKLOADS); any other
shape can be drawn with `random_problem`.

Recipe (fixed so that every run and every consumer sees the same bits):
  rng = numpy.random.default_rng(seed); draw the layout first, then W as
  (nnz, b, b), then x, then dy, then (grouped weight gradient only) x_t, dy_t for
  t = 1 .. G-1.  Every array is drawn in its stored layout as float32
  standard_normal, scaled, and cast to the storage dtype with round-to-nearest-even
  (torch's .to()).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass
class Workload:
    name: str
    hidden: int          # C = K
    block: int           # b
    N: int               # minibatch
    fa: int              # feature_axis: 1 -> (N, C), 0 -> (C, N)
    dtypes: tuple        # storage dtypes the workload is run in
    G: int               # steps summed by the grouped weight gradient
    layout_kind: str
    w_std: Optional[float]  # None: fan-in scaling 1/sqrt(32 * mean blocks per column)
    seed: int


# Seeds are 1000 + i for the i-th workload.
WORKLOADS = {
    "tiny": Workload("tiny", 256, 32, 64, 1, ("f32",), 1, "bern0.5", None, 1000),
    "hidden4096_b32_n64": Workload("hidden4096_b32_n64", 4096, 32, 64, 1, ("f32", "bf16"), 1,
                                   "bern0.5", 0.02, 1001),
    "hidden4096_b16_n512": Workload("hidden4096_b16_n512", 4096, 16, 512, 0, ("f16",), 1,
                                    "bern0.25_cover", 0.02, 1002),
    "hidden8192_b8_n1024": Workload("hidden8192_b8_n1024", 8192, 8, 1024, 0, ("bf16",), 1,
                                    "bern0.1_diag", 0.02, 1003),
    "hidden8192_b32_n4096_g8": Workload("hidden8192_b32_n4096_g8", 8192, 32, 4096, 1, ("bf16",), 8,
                                        "band_random3pct", 0.02, 1004),
    # Supplementary: the same dimensions at half density, so that the contraction (not
    # the activation stream) bounds every pass; large-N dense-block matrix-core shape.
    "hidden8192_b32_n4096_dense50": Workload("hidden8192_b32_n4096_dense50", 8192, 32, 4096, 1,
                                             ("bf16",), 1, "bern0.5_diag", 0.02, 1005),
}
WORKLOAD_ORDER = list(WORKLOADS)


def make_layout(kind: str, R: int, S: int, rng: np.random.Generator) -> np.ndarray:
    """A 0/1 block layout of shape (R, S) as uint8, row = input block c, column = output block k."""
    if kind.startswith("bern") and kind[4:].replace(".", "").isdigit():
        p = float(kind[4:])
        return (rng.random((R, S)) < p).astype(np.uint8)
    if kind == "bern0.25_cover":
        # Bernoulli(0.25), then every empty row (ascending) gets one random block, then
        # every empty column (ascending) gets one random block.
        L = (rng.random((R, S)) < 0.25).astype(np.uint8)
        for r in range(R):
            if not L[r].any():
                L[r, rng.integers(S)] = 1
        for k in range(S):
            if not L[:, k].any():
                L[rng.integers(R), k] = 1
        return L
    if kind.startswith("bern") and kind.endswith("_diag"):
        L = (rng.random((R, S)) < float(kind[4:-5]))
        d = min(R, S)
        L[np.arange(d), np.arange(d)] = True
        return L.astype(np.uint8)
    if kind == "band_random3pct":
        # Diagonal plus the four off-diagonals with 0 < |c-k| <= 2, then distinct random
        # off-band cells until the density is round(0.03 * R * S).
        assert R == S
        c, k = np.meshgrid(np.arange(R), np.arange(S), indexing="ij")
        band = np.abs(c - k) <= 2
        L = band.copy()
        target = int(round(0.03 * R * S))
        extra = target - int(band.sum())
        off = np.flatnonzero(~band.ravel())
        pick = rng.choice(off, size=max(extra, 0), replace=False)
        L.ravel()[pick] = True
        return L.astype(np.uint8)
    raise ValueError(f"unknown layout kind {kind!r}")


def _draw(rng, shape, scale, dtype) -> torch.Tensor:
    a = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return torch.from_numpy(a).to(DTYPES[dtype])


@dataclasses.dataclass
class Problem:
    layout: np.ndarray      # uint8 (R, S)
    block: int
    fa: int
    N: int
    dtype: str
    w: torch.Tensor         # (nnz, b, b), CPU, storage dtype
    xs: List[torch.Tensor]  # G activations, stored layout
    dys: List[torch.Tensor]  # G output gradients, stored layout

    @property
    def R(self):
        return self.layout.shape[0]

    @property
    def S(self):
        return self.layout.shape[1]

    @property
    def nnz(self):
        return int(self.layout.sum())


def act_shape(fa: int, N: int, F: int):
    return (N, F) if fa == 1 else (F, N)


def random_problem(rng: np.random.Generator, layout: np.ndarray, block: int, N: int, fa: int,
                   dtype: str, G: int = 1, w_std: float = 0.02, x_std: float = 1.0) -> Problem:
    """Draw W, x, dy (and G-1 further x_t, dy_t) for a given layout, in the recipe's order."""
    layout = np.ascontiguousarray(layout, dtype=np.uint8)
    R, S = layout.shape
    nnz = int(layout.sum())
    w = _draw(rng, (nnz, block, block), w_std, dtype)
    xs, dys = [], []
    for _ in range(G):
        xs.append(_draw(rng, act_shape(fa, N, R * block), x_std, dtype))
        dys.append(_draw(rng, act_shape(fa, N, S * block), 1.0, dtype))
    return Problem(layout, block, fa, N, dtype, w, xs, dys)


def workload_problem(name: str, dtype: Optional[str] = None, N: Optional[int] = None,
                     G: Optional[int] = None) -> Problem:
    """The named workload's seeded inputs (layout, W, x, dy, and the grouped steps)."""
    wl = WORKLOADS[name]
    dtype = dtype or wl.dtypes[0]
    rng = np.random.default_rng(wl.seed)
    R = S = wl.hidden // wl.block
    layout = make_layout(wl.layout_kind, R, S, rng)
    nnz = int(layout.sum())
    if wl.w_std is None:
        w_std = 1.0 / np.sqrt(32.0 * nnz / S)
    else:
        w_std = wl.w_std
    return random_problem(rng, layout, wl.block, N or wl.N, wl.fa, dtype, G or wl.G, w_std)


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a CPU tensor as numpy: float32 stays float32, 16-bit types become uint16."""
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


@dataclasses.dataclass
class NormProblem:
    """Seeded inputs of a layer norm over the feature axis (x and dy in the activation
    layout of `axis`: (N, C) for 1, (C, N) for 0; g and b float32 (C,))."""
    N: int
    C: int
    axis: int
    dtype: str
    x: torch.Tensor
    dy: torch.Tensor
    g: torch.Tensor
    b: torch.Tensor


def norm_problem(rng: np.random.Generator, N: int, C: int, axis: int, dtype: str,
                 relu_margin: bool = False) -> NormProblem:
    """x ~ N(shift, scale) per vector (shift and scale drawn per vector), dy ~ N(0, 1),
    g ~ N(1, 0.25), b ~ N(0, 0.25).  With relu_margin, |g| <= 0.25 and |b| >= 2, so
    g*xhat + b keeps the sign of b while |xhat| < 8 (no value near the ReLU's kink)."""
    shape = act_shape(axis, N, C)
    shift = rng.standard_normal(N).astype(np.float32) * 2
    scale = (0.5 + rng.random(N)).astype(np.float32)
    z = rng.standard_normal(shape).astype(np.float32)
    xv = z * (scale[:, None] if axis == 1 else scale[None, :]) + (shift[:, None] if axis == 1 else shift[None, :])
    x = torch.from_numpy(xv).to(DTYPES[dtype])
    dy = _draw(rng, shape, 1.0, dtype)
    if relu_margin:
        g = (rng.random(C).astype(np.float32) - 0.5) * 0.5
        b = (2 + rng.random(C).astype(np.float32)) * np.where(rng.random(C) < 0.5, -1, 1).astype(np.float32)
    else:
        g = (1 + 0.25 * rng.standard_normal(C)).astype(np.float32)
        b = (0.25 * rng.standard_normal(C)).astype(np.float32)
    return NormProblem(N, C, axis, dtype, x, dy, torch.from_numpy(g), torch.from_numpy(b))


@dataclasses.dataclass
class ProjProblem:
    """Seeded inputs of SparseProj: x, a (dense, nhidden features), s (projected, nproj
    features), in the activation layout of fa ((N, F) for 1, (F, N) for 0); lut the
    feature map (None: the blocked default of the given proj_stride / block_size)."""
    N: int
    nhidden: int
    nproj: int
    fa: int
    dtype: str
    lut: Optional[np.ndarray]
    x: torch.Tensor
    a: torch.Tensor
    s: torch.Tensor


def proj_problem(rng: np.random.Generator, N: int, nhidden: int, nproj: int, fa: int, dtype: str,
                 random_map: bool) -> ProjProblem:
    """random_map: nproj distinct dense features in random order (rng.permutation), drawn
    first; else lut is None (the blocked default).  Then x, a ~ N(0, 1) dense and
    s ~ N(0, 1) projected."""
    lut = rng.permutation(nhidden)[:nproj].astype(np.int64) if random_map else None
    x = _draw(rng, act_shape(fa, N, nhidden), 1.0, dtype)
    a = _draw(rng, act_shape(fa, N, nhidden), 1.0, dtype)
    s = _draw(rng, act_shape(fa, N, nproj), 1.0, dtype)
    return ProjProblem(N, nhidden, nproj, fa, dtype, lut, x, a, s)


@dataclasses.dataclass
class ConvProblem:
    """Seeded inputs of BlocksparseConv: BCK (one (input channels, output channels) pair
    per block), filter F (nblocks, Bc, *TRS, Bk), input I (N, C, *DHW) and output
    gradient dO (N, K, *MPQ)."""
    BCK: list
    F: torch.Tensor
    I: torch.Tensor
    dO: torch.Tensor


def conv_problem(rng: np.random.Generator, N: int, C: int, K: int, Bc: int, Bk: int, nblocks: int, TRS, DHW, MPQ,
                 dtype: str, f_std: float = 0.1, contiguous_blocks: bool = False) -> ConvProblem:
    """Channel lists first (contiguous_blocks: block b takes the b-th (c-block, k-block)
    pair of a random choice of distinct cells of the (C/Bc) x (K/Bk) block grid, with
    consecutive channels; else rng.permutation draws per block, so blocks may share
    channels), then F ~ N(0, f_std), I ~ N(0, 1), dO ~ N(0, 1)."""
    if contiguous_blocks:
        cells = rng.choice((C // Bc) * (K // Bk), nblocks, replace=False)
        BCK = [(tuple(range((c // (K // Bk)) * Bc, (c // (K // Bk)) * Bc + Bc)),
                tuple(range((c % (K // Bk)) * Bk, (c % (K // Bk)) * Bk + Bk))) for c in sorted(cells)]
    else:
        BCK = [(tuple(int(v) for v in rng.permutation(C)[:Bc]), tuple(int(v) for v in rng.permutation(K)[:Bk]))
               for _ in range(nblocks)]
    F = _draw(rng, (nblocks, Bc) + tuple(TRS) + (Bk,), f_std, dtype)
    I = _draw(rng, (N, C) + tuple(DHW), 1.0, dtype)
    dO = _draw(rng, (N, K) + tuple(MPQ), 1.0, dtype)
    return ConvProblem(BCK, F, I, dO)
