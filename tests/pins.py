"""Pins for the CPU oracle: checks against facts fixed by the pages and by mathematics.

Each pin takes an oracle library handle (so the same pins can be run against
deliberately broken builds of the oracle, see test_oracle_mutants.py) and raises
AssertionError when the oracle disagrees with:
  * a library routine (numpy float64 matmul of the layout-masked dense weight,
    assembled here by a separate scatter in numpy's row-major nonzero order);
  * closed forms (all-ones layout = dense GEMM; the usage example's x = ones
    gives the weight's column sums in every row; identity_init reproduces x);
  * algebraic identities (adjoints, the transposed plan, grouping);
  * exhaustive brute force on tiny layouts with scalar Python loops;
  * exact decoding of every 16-bit pattern (numpy float16, torch bfloat16).
None of these calls the oracle to produce an expected value.
"""
from __future__ import annotations

import itertools

import numpy as np
import torch

import oracle
import synth

DT_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def to64(t: torch.Tensor) -> np.ndarray:
    return t.double().numpy()


def dense_w(layout: np.ndarray, w64: np.ndarray) -> np.ndarray:
    """W~ (C x K): block t of w64 placed at the t-th nonzero of the layout in row-major order."""
    R, S = layout.shape
    b = w64.shape[1]
    Wd = np.zeros((R * b, S * b))
    cs, ks = np.nonzero(layout)
    for t, (c, k) in enumerate(zip(cs, ks)):
        Wd[c * b:(c + 1) * b, k * b:(k + 1) * b] = w64[t]
    return Wd


def rel(a, b):
    m = np.max(np.abs(b)) if b.size else 0.0
    d = np.max(np.abs(a - b)) if a.size else 0.0
    return d / m if m > 0 else d


def _problem(seed, R, S, b, N, fa, dtype, G=1, density=0.5):
    rng = np.random.default_rng(seed)
    L = (rng.random((R, S)) < density).astype(np.uint8)
    return synth.random_problem(rng, L, b, N, fa, dtype, G=G, w_std=0.3)


def _bits(t):
    return synth.to_bits(t)


# ----------------------------------------------------------------------------------
def pin_decode_f16(lib):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = _decode_with(lib, pats, "f16")
    ref = pats.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def pin_decode_bf16(lib):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = _decode_with(lib, pats, "bf16")
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _decode_with(lib, pats, dtype):
    lib = lib or oracle.load()
    import ctypes
    out = np.empty(pats.size, dtype=np.float64)
    p = pats.ctypes.data_as(ctypes.c_void_p)
    for t in range(pats.size):
        out[t] = lib.orc_decode(p, t, oracle.DT[dtype])
    return out


# ----------------------------------------------------------------------------------
def pin_dense_masked(lib, b=8, fa=1, dtype="f32", R=3, S=5, N=7, seed=0):
    """All three passes against numpy fp64 matmuls of the masked dense weight."""
    P = _problem(seed, R, S, b, N, fa, dtype, G=2)
    L = P.layout
    Wd = dense_w(L, to64(P.w))
    x64 = [to64(t) for t in P.xs]
    dy64 = [to64(t) for t in P.dys]
    X = [a if fa == 1 else a.T for a in x64]     # (N, C)
    DY = [a if fa == 1 else a.T for a in dy64]   # (N, K)
    y = oracle.fprop(L, b, fa, _bits(P.xs[0]), _bits(P.w), N, dtype, lib=lib)
    yref = X[0] @ Wd
    assert rel(y if fa == 1 else y.T, yref) < 1e-12, "fprop"
    dx = oracle.bprop(L, b, fa, _bits(P.dys[0]), _bits(P.w), N, dtype, lib=lib)
    dxref = DY[0] @ Wd.T
    assert rel(dx if fa == 1 else dx.T, dxref) < 1e-12, "bprop"
    dw = oracle.updat(L, b, fa, [_bits(t) for t in P.xs], [_bits(t) for t in P.dys], N, dtype, lib=lib)
    full = sum(X[g].T @ DY[g] for g in range(2))    # (C, K)
    mask = np.kron(L, np.ones((b, b)))
    assert np.all(dense_w(L, dw)[mask == 0] == 0)
    ref_blocks = np.stack([full[c * b:(c + 1) * b, k * b:(k + 1) * b] for c, k in zip(*np.nonzero(L))]) \
        if L.sum() else np.zeros((0, b, b))
    assert rel(dw, ref_blocks) < 1e-12, "updat"


def pin_all_ones_is_dense(lib, b=8, fa=1, R=3, S=4, N=5, seed=1):
    """All-ones layout: the op is the textbook dense GEMM x . W with W = blocks tiled in id order."""
    rng = np.random.default_rng(seed)
    L = np.ones((R, S), dtype=np.uint8)
    P = synth.random_problem(rng, L, b, N, fa, "f32", w_std=0.3)
    w = to64(P.w)
    # ids of an all-ones layout are c*S + k; tile them by reshaping.
    Wd = w.reshape(R, S, b, b).transpose(0, 2, 1, 3).reshape(R * b, S * b)
    X = to64(P.xs[0]) if fa == 1 else to64(P.xs[0]).T
    y = oracle.fprop(L, b, fa, _bits(P.xs[0]), _bits(P.w), N, lib=lib)
    assert rel(y if fa == 1 else y.T, X @ Wd) < 1e-12


def pin_ones_input_gives_column_sums(lib, b=16, R=4, S=3, N=6, seed=2):
    """The usage example feeds x = ones: every row of y is the column sums of W~."""
    rng = np.random.default_rng(seed)
    L = (rng.random((R, S)) < 0.6).astype(np.uint8)
    L[0, 0] = 1
    P = synth.random_problem(rng, L, b, N, 1, "f32", w_std=0.3)
    x = np.ones((N, R * b), dtype=np.float32)
    y = oracle.fprop(L, b, 1, x, _bits(P.w), N, lib=lib)
    w = to64(P.w)
    colsum = np.zeros(S * b)
    for t, (c, k) in enumerate(zip(*np.nonzero(L))):
        colsum[k * b:(k + 1) * b] += w[t].sum(axis=0)
    for n in range(N):
        assert rel(y[n], colsum) < 1e-12


def pin_identity(lib, b=8, R=4, S=4, N=5, seed=3):
    """identity_init: identity on present diagonal blocks; then y = x there and 0 elsewhere."""
    rng = np.random.default_rng(seed)
    L = (rng.random((R, S)) < 0.5).astype(np.uint8)
    L[1, 1] = 1
    L[2, 2] = 0
    w = oracle.identity(L, b, lib=lib)
    for t, (c, k) in enumerate(zip(*np.nonzero(L))):
        assert np.array_equal(w[t], np.eye(b) if c == k else np.zeros((b, b)))
    x = rng.standard_normal((N, R * b)).astype(np.float32)
    y = oracle.fprop(L, b, 1, x, w.astype(np.float32), N, lib=lib)
    for k in range(S):
        sl = slice(k * b, (k + 1) * b)
        if L[k, k]:
            assert np.array_equal(y[:, sl], x[:, sl].astype(np.float64))
        else:
            assert np.all(y[:, sl] == 0)
    dx = oracle.bprop(L, b, 1, x, w.astype(np.float32), N, lib=lib)
    for c in range(R):
        sl = slice(c * b, (c + 1) * b)
        if L[c, c]:
            assert np.array_equal(dx[:, sl], x[:, sl].astype(np.float64))
        else:
            assert np.all(dx[:, sl] == 0)


def pin_block_coord(lib, R=5, S=7, seed=4):
    rng = np.random.default_rng(seed)
    L = (rng.random((R, S)) < 0.4).astype(np.uint8)
    for t, (c, k) in enumerate(zip(*np.nonzero(L))):
        assert oracle.block_coord(L, t, lib=lib) == (c, k)


def pin_adjoints(lib, b=16, fa=0, R=3, S=4, N=9, seed=5):
    """<fprop(x), dy> = <x, bprop(dy)> and <updat(x, dy), V> = <fprop_V(x), dy>."""
    P = _problem(seed, R, S, b, N, fa, "f32")
    L = P.layout
    xb, dyb, wb = _bits(P.xs[0]), _bits(P.dys[0]), _bits(P.w)
    y = oracle.fprop(L, b, fa, xb, wb, N, lib=lib)
    dx = oracle.bprop(L, b, fa, dyb, wb, N, lib=lib)
    lhs = float(np.sum(y * to64(P.dys[0])))
    rhs = float(np.sum(to64(P.xs[0]) * dx))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)) * 100
    dw = oracle.updat(L, b, fa, [xb], [dyb], N, lib=lib)
    V = np.random.default_rng(seed + 1).standard_normal(dw.shape).astype(np.float32)
    yV = oracle.fprop(L, b, fa, xb, V, N, lib=lib)
    lhs = float(np.sum(dw * V.astype(np.float64)))
    rhs = float(np.sum(yV * to64(P.dys[0])))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)) * 100


def pin_transposed_plan(lib, b=8, fa=1, R=3, S=5, N=4, seed=6):
    """bprop under (L, W) equals fprop under (L^T, W^T re-numbered by L^T's row-major ids)."""
    P = _problem(seed, R, S, b, N, fa, "f32")
    L = P.layout
    w = _bits(P.w)
    LT = np.ascontiguousarray(L.T)
    id_of = -np.ones((R, S), dtype=np.int64)
    for t, (c, k) in enumerate(zip(*np.nonzero(L))):
        id_of[c, k] = t
    wT = np.stack([w[id_of[c, k]].T for k, c in zip(*np.nonzero(LT))]) if L.sum() else w
    wT = np.ascontiguousarray(wT)
    dx = oracle.bprop(L, b, fa, _bits(P.dys[0]), w, N, lib=lib)
    y2 = oracle.fprop(LT, b, fa, _bits(P.dys[0]), wT, N, lib=lib)
    assert np.array_equal(dx, y2)


def pin_grouping(lib, b=8, fa=1, R=2, S=3, N=5, G=3, seed=7):
    """Grouped dW = sum of single-step dWs = one dW over the concatenated minibatch."""
    P = _problem(seed, R, S, b, N, fa, "f32", G=G, density=0.7)
    L = P.layout
    xs = [_bits(t) for t in P.xs]
    dys = [_bits(t) for t in P.dys]
    g = oracle.updat(L, b, fa, xs, dys, N, lib=lib)
    singles = sum(oracle.updat(L, b, fa, [xs[t]], [dys[t]], N, lib=lib) for t in range(G))
    assert rel(g, singles) < 1e-13
    ax = 0 if fa == 1 else 1
    xc = np.ascontiguousarray(np.concatenate(xs, axis=ax))
    dyc = np.ascontiguousarray(np.concatenate(dys, axis=ax))
    cat = oracle.updat(L, b, fa, [xc], [dyc], N * G, lib=lib)
    assert rel(g, cat) < 1e-13
    sub = oracle.updat(L, b, fa, xs, dys, N, ids=[int(L.sum()) - 1, 0], lib=lib)
    assert np.array_equal(sub[0], g[-1]) and np.array_equal(sub[1], g[0])


def pin_accumulate(lib, b=8, fa=0, R=3, S=4, N=6, seed=12):
    """Accumulating updat: onto zeros it is the plain weight gradient; a sequence of 7
    steps split into groups of 3 and 4 and accumulated equals the 7-step sum (up to the
    fp32 rounding of the stored partial); a bf16 / f16 stored gradient enters with the
    value torch's own conversion gives its bits."""
    P = _problem(seed, R, S, b, N, fa, "f32", G=7, density=0.6)
    L = P.layout
    xs = [_bits(t) for t in P.xs]
    dys = [_bits(t) for t in P.dys]
    nz = int(L.sum())
    zero = np.zeros((nz, b, b), np.float32)
    assert np.array_equal(oracle.updat_accumulate(L, b, fa, zero, "f32", xs[:3], dys[:3], N, lib=lib),
                          oracle.updat(L, b, fa, xs[:3], dys[:3], N, lib=lib))
    part = oracle.updat(L, b, fa, xs[:3], dys[:3], N, lib=lib).astype(np.float32)
    whole = oracle.updat(L, b, fa, xs, dys, N, lib=lib)
    acc = oracle.updat_accumulate(L, b, fa, part, "f32", xs[3:], dys[3:], N, lib=lib)
    assert rel(acc, whole) < 1e-6
    single = oracle.updat(L, b, fa, xs[3:], dys[3:], N, lib=lib)
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        stored = torch.from_numpy(part).to(tdt)
        got = oracle.updat_accumulate(L, b, fa, _bits(stored), dt, xs[3:], dys[3:], N, lib=lib)
        assert rel(got - single, to64(stored)) < 1e-12


def pin_one_hot_rows(lib, b=8, R=3, S=3, seed=8):
    """x rows one-hot on distinct features: dW row (c, i) of block (c, k) copies dy's row for that feature."""
    rng = np.random.default_rng(seed)
    L = (rng.random((R, S)) < 0.6).astype(np.uint8)
    L[0, 1] = 1
    C, K = R * b, S * b
    N = C
    perm = rng.permutation(C)
    x = np.zeros((N, C), dtype=np.float32)
    x[np.arange(N), perm] = 1.0
    dy = rng.standard_normal((N, K)).astype(np.float32)
    dw = oracle.updat(L, b, 1, [x], [dy], N, lib=lib)
    inv = np.argsort(perm)   # feature f is hot in row inv[f]
    for t, (c, k) in enumerate(zip(*np.nonzero(L))):
        for i in range(b):
            assert np.array_equal(dw[t][i], dy[inv[c * b + i], k * b:(k + 1) * b].astype(np.float64))


def pin_feature_axis(lib, b=16, R=2, S=3, N=6, seed=9, dtype="bf16"):
    """feature_axis=0 is feature_axis=1 on transposed activations, for all three passes."""
    P = _problem(seed, R, S, b, N, 1, dtype)
    L = P.layout
    x1, dy1, w = _bits(P.xs[0]), _bits(P.dys[0]), _bits(P.w)
    x0, dy0 = np.ascontiguousarray(x1.T), np.ascontiguousarray(dy1.T)
    assert np.array_equal(oracle.fprop(L, b, 1, x1, w, N, dtype, lib=lib),
                          oracle.fprop(L, b, 0, x0, w, N, dtype, lib=lib).T)
    assert np.array_equal(oracle.bprop(L, b, 1, dy1, w, N, dtype, lib=lib),
                          oracle.bprop(L, b, 0, dy0, w, N, dtype, lib=lib).T)
    assert np.array_equal(oracle.updat(L, b, 1, [x1], [dy1], N, dtype, lib=lib),
                          oracle.updat(L, b, 0, [x0], [dy0], N, dtype, lib=lib))


def _scalar_dense(L, b, w64):
    R, S = L.shape
    C, K = R * b, S * b
    Wd = [[0.0] * K for _ in range(C)]
    t = 0
    for c in range(R):
        for k in range(S):
            if L[c][k]:
                for i in range(b):
                    for j in range(b):
                        Wd[c * b + i][k * b + j] = float(w64[t][i][j])
                t += 1
    return Wd


def pin_bruteforce_tiny(lib, b=2, N=2, seed=10):
    """Every layout of every grid up to 3x3, against scalar Python loops over the dense definition."""
    rng = np.random.default_rng(seed)
    for R, S in [(1, 1), (1, 2), (2, 1), (2, 2), (2, 3), (3, 2), (3, 3)]:
        C, K = R * b, S * b
        for bits in itertools.product([0, 1], repeat=R * S):
            L = np.array(bits, dtype=np.uint8).reshape(R, S)
            nnz = int(L.sum())
            w = rng.integers(-3, 4, size=(nnz, b, b)).astype(np.float32)
            x = rng.integers(-3, 4, size=(N, C)).astype(np.float32)
            dy = rng.integers(-3, 4, size=(N, K)).astype(np.float32)
            Wd = _scalar_dense(L, b, w)
            y = oracle.fprop(L, b, 1, x, w, N, lib=lib)
            dx = oracle.bprop(L, b, 1, dy, w, N, lib=lib)
            dw = oracle.updat(L, b, 1, [x], [dy], N, lib=lib)
            for n in range(N):
                for f in range(K):
                    assert y[n, f] == sum(float(x[n, g]) * Wd[g][f] for g in range(C))
                for g in range(C):
                    assert dx[n, g] == sum(float(dy[n, f]) * Wd[g][f] for f in range(K))
            t = 0
            for c in range(R):
                for k in range(S):
                    if L[c, k]:
                        for i in range(b):
                            for j in range(b):
                                ref = sum(float(x[n, c * b + i]) * float(dy[n, k * b + j]) for n in range(N))
                                assert dw[t, i, j] == ref
                        t += 1


ALL_PINS = [
    pin_decode_f16, pin_decode_bf16, pin_dense_masked, pin_all_ones_is_dense,
    pin_ones_input_gives_column_sums, pin_identity, pin_block_coord, pin_adjoints,
    pin_transposed_plan, pin_grouping, pin_accumulate, pin_one_hot_rows, pin_feature_axis, pin_bruteforce_tiny,
]
