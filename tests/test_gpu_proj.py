"""SparseProj on the GPU against the CPU oracle (calls through the C ABI).

Copies (gather, scatter, and the untouched features of scatter_add / scatter_mul) are
compared bit for bit; add and mul, rounded once from fp32 to the storage type, within
the floating-point tolerance (and almost all elements identical).  Cases: both feature
axes, all three dtypes, the blocked default map (16-byte vector path) and random maps
(element path), widths and minibatches that are not multiples of 16 bytes, in-place
scatter_add, and the autograd backward of every op."""
import numpy as np
import pytest
import torch

import block_sparse_matrix_amd as bs
import synth
from gpu_util import TOL, assert_close, dev
from oracle import sparse_proj as sp

pytestmark = pytest.mark.gpu


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def _bits_equal(got: torch.Tensor, ref: np.ndarray, dtype: str) -> bool:
    r = torch.from_numpy(ref).to(synth.DTYPES[dtype])
    return torch.equal(got.cpu().view(torch.int16 if dtype != "f32" else torch.int32),
                       r.view(torch.int16 if dtype != "f32" else torch.int32))


CASES = [
    # N, nhidden, nproj, proj_stride, block_size, random map
    (64, 512, 256, 64, 32, False),
    (37, 520, 256, 64, 32, False),
    (48, 200, 72, None, 8, False),
    (33, 300, 77, None, None, True),
    (16, 4096, 1000, None, None, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"N{c[0]}-H{c[1]}-P{c[2]}-{'rand' if c[5] else 'blk'}" for c in CASES])
@pytest.mark.parametrize("fa", [1, 0])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_ops(case, fa, dtype):
    N, H, Pn, stride, bsz, rnd = case
    print(f"case proj N={N} H={H} P={Pn} fa={fa} {dtype} random={rnd}", flush=True)
    rng = np.random.default_rng(N + H + Pn + fa)
    P = synth.proj_problem(rng, N, H, Pn, fa, dtype, rnd)
    proj = bs.SparseProj(H, Pn, stride, bsz or 32, gather_lut=P.lut, feature_axis=fa)
    # the oracle takes the map from the inputs (the given map, or the oracle's own
    # default), never from the library; the library's copy must equal it
    lut = sp.check_lut(P.lut, H) if P.lut is not None else sp.default_lut(H, Pn, stride, bsz or 32)
    assert np.array_equal(proj.gather_lut.astype(np.int64), lut)
    x, a, s = dev(P.x), dev(P.a), dev(P.s)
    g = proj.gather(x)
    sc = proj.scatter(s)
    za = proj.scatter_add(x, s)
    zm = proj.scatter_mul(x, s)
    gm = proj._gather_mul(x, a)
    torch.cuda.synchronize()
    X, A, S = _f64(P.x), _f64(P.a), _f64(P.s)
    assert _bits_equal(g, sp.gather(lut, X, fa), dtype)
    assert _bits_equal(sc, sp.scatter(lut, S, H, fa), dtype)
    for got, ref, what in ((za, sp.scatter_add(lut, X, S, fa), "scatter_add"),
                           (zm, sp.scatter_mul(lut, X, S, fa), "scatter_mul"),
                           (gm, sp.gather_mul(lut, X, A, fa), "gather_mul")):
        assert_close(got, ref, dtype, what)
        same = (got.cpu() == torch.from_numpy(ref).to(synth.DTYPES[dtype])).double().mean().item()
        assert same > 0.999, f"{what}: only {same:.4f} of the elements equal the rounded oracle"
    # features outside the map pass through scatter_add / scatter_mul bit for bit
    keep = np.setdiff1d(np.arange(H), lut)
    if keep.size:
        idx = torch.from_numpy(keep).cuda()
        fdim = 1 if fa == 1 else 0
        for z in (za, zm):
            assert torch.equal(z.index_select(fdim, idx), x.index_select(fdim, idx))


@pytest.mark.parametrize("fa", [1, 0])
def test_scatter_add_in_place(fa):
    rng = np.random.default_rng(5 + fa)
    P = synth.proj_problem(rng, 40, 256, 96, fa, "bf16", True)
    proj = bs.SparseProj(256, gather_lut=P.lut, feature_axis=fa)
    x, s = dev(P.x), dev(P.s)
    ref = proj.scatter_add(x, s)
    bs.bsmm_proj_scatter_add(proj.handle, x, s, x, 40, fa)   # z = x
    torch.cuda.synchronize()
    assert torch.equal(x, ref)


@pytest.mark.parametrize("fa", [1, 0])
def test_autograd(fa):
    """Backward of each op against the oracle: d gather = scatter, d scatter = gather,
    d scatter_add = (dz, gather(dz)), d scatter_mul = (scatter_mul(dz, y), gather_mul(dz, x))."""
    rng = np.random.default_rng(11 + fa)
    N, H, Pn = 24, 160, 48
    P = synth.proj_problem(rng, N, H, Pn, fa, "f32", True)
    proj = bs.SparseProj(H, gather_lut=P.lut, feature_axis=fa)
    lut = P.lut
    dz = synth.proj_problem(rng, N, H, Pn, fa, "f32", False)
    dzh, dzp = dev(dz.x), dev(dz.s)
    X, S, DH, DP = _f64(P.x), _f64(P.s), _f64(dz.x), _f64(dz.s)

    x = dev(P.x).requires_grad_()
    proj.gather(x).backward(dzp)
    assert_close(x.grad, sp.scatter(lut, DP, H, fa), "f32", "d gather")
    s = dev(P.s).requires_grad_()
    proj.scatter(s).backward(dzh)
    assert_close(s.grad, sp.gather(lut, DH, fa), "f32", "d scatter")
    x = dev(P.x).requires_grad_()
    s = dev(P.s).requires_grad_()
    proj.scatter_add(x, s).backward(dzh)
    assert torch.equal(x.grad, dzh)
    assert_close(s.grad, sp.gather(lut, DH, fa), "f32", "d scatter_add / y")
    x = dev(P.x).requires_grad_()
    s = dev(P.s).requires_grad_()
    proj.scatter_mul(x, s).backward(dzh)
    assert_close(x.grad, sp.scatter_mul(lut, DH, S, fa), "f32", "d scatter_mul / x")
    assert_close(s.grad, sp.gather_mul(lut, DH, X, fa), "f32", "d scatter_mul / y")


def test_bench_configuration_full_size():
    """The configuration bench.py times (nhidden 8192 -> nproj 4096 in blocks of 32 every
    64 features, N = 4096, bf16, features last, the same seed), all five ops against the
    oracle: copies bit for bit, add / mul to the dtype gate.  The map is the oracle's
    default map for these arguments."""
    N, H, Pn = 4096, 8192, 4096
    print(f"case proj full size N={N} H={H} P={Pn} bf16", flush=True)
    P = synth.proj_problem(np.random.default_rng(17), N, H, Pn, 1, "bf16", False)
    proj = bs.SparseProj(H, Pn, 64, 32)
    lut = sp.default_lut(H, Pn, 64, 32)
    assert np.array_equal(proj.gather_lut.astype(np.int64), lut)
    x, a, s = dev(P.x), dev(P.a), dev(P.s)
    g = proj.gather(x)
    sc = proj.scatter(s)
    za = proj.scatter_add(x, s)
    zm = proj.scatter_mul(x, s)
    gm = proj._gather_mul(x, a)
    torch.cuda.synchronize()
    X, A, S = _f64(P.x), _f64(P.a), _f64(P.s)
    assert _bits_equal(g, sp.gather(lut, X, 1), "bf16")
    assert _bits_equal(sc, sp.scatter(lut, S, H, 1), "bf16")
    assert_close(za, sp.scatter_add(lut, X, S, 1), "bf16", "scatter_add")
    assert_close(zm, sp.scatter_mul(lut, X, S, 1), "bf16", "scatter_mul")
    assert_close(gm, sp.gather_mul(lut, X, A, 1), "bf16", "gather_mul")
