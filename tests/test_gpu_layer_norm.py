"""GPU parity of layer_norm (forward and gradient) against the float64 oracle, through
the C ABI: both feature axes, fp32/bf16/f16 storage, with and without the ReLU, the
16-byte-vector and one-value paths (ragged and unaligned widths), one-vector and
one-feature edge cases, and the full N = 4096, C = 8192 activation of the band
workload."""
import numpy as np
import pytest
import torch

import block_sparse_matrix_amd as bs
import synth
from gpu_util import TOL, assert_close, dev, rel_err
from oracle import layer_norm as oln

pytestmark = pytest.mark.gpu

SHAPES = [(37, 1000), (5, 8192), (64, 24), (3, 3), (1, 17), (130, 16384), (300, 264), (2, 1)]


def _run(N, C, axis, dtype, relu, seed, check_grad=True):
    print(f"case layer_norm N={N} C={C} axis={axis} dtype={dtype} relu={relu}", flush=True)
    rng = np.random.default_rng(seed)
    P = synth.norm_problem(rng, N, C, axis, dtype, relu_margin=relu)
    x, dy, g, b = dev(P.x), dev(P.dy), dev(P.g), dev(P.b)
    y = torch.empty_like(x)
    mean = torch.empty(N, device="cuda")
    rstd = torch.empty(N, device="cuda")
    bs.bsmm_layer_norm(x, g, b, y, mean, rstd, axis, 1e-6, relu)
    torch.cuda.synchronize()
    xb, dyb = synth.to_bits(P.x), synth.to_bits(P.dy)
    ry, rmean, rrstd = oln.layer_norm(xb, P.g.numpy(), P.b.numpy(), axis, 1e-6, relu, dtype)
    if relu:   # the ReLU mask must not depend on rounding (see synth.norm_problem)
        xr = oln.decode(xb, dtype)
        xr = xr if axis == 1 else xr.T
        assert np.abs((xr - rmean[:, None]) * rrstd[:, None]).max() < 8
    assert_close(y, ry, dtype, "layer_norm y")
    assert rel_err(mean, rmean) <= 1e-5 and rel_err(rstd, rrstd) <= 1e-5
    if not check_grad:
        return
    dx = torch.empty_like(x)
    dg = torch.empty_like(g)
    db = torch.empty_like(b)
    bs.bsmm_layer_norm_grad(dy, x, g, b, mean, rstd, dx, dg, db, axis, relu)
    torch.cuda.synchronize()
    rdx, rdg, rdb = oln.layer_norm_grad(dyb, xb, P.g.numpy(), P.b.numpy(), axis, 1e-6, relu, dtype)
    assert_close(dx, rdx, dtype, "layer_norm dx")
    assert rel_err(dg, rdg) <= 1e-5, ("dg", rel_err(dg, rdg))
    assert rel_err(db, rdb) <= 1e-5, ("db", rel_err(db, rdb))


@pytest.mark.parametrize("relu", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("N,C", SHAPES)
def test_layer_norm(N, C, axis, dtype, relu):
    if axis == 1 and dtype == "f32" and C > 8192:
        with pytest.raises(bs.BsmmError):
            _run(N, C, axis, dtype, relu, 0)
        return
    _run(N, C, axis, dtype, relu, N * 7 + C + axis)


def test_layer_norm_unaligned_params():
    """g and b not 16-byte aligned: the one-value path reads them (axis 1)."""
    N, C, dtype = 9, 512, "bf16"
    print(f"case layer_norm unaligned params N={N} C={C}", flush=True)
    P = synth.norm_problem(np.random.default_rng(11), N, C, 1, dtype)
    x = dev(P.x)
    gb = torch.empty(2 * C + 2, device="cuda")
    g, b = gb[1:C + 1], gb[C + 1:2 * C + 1]
    g.copy_(P.g.cuda())
    b.copy_(P.b.cuda())
    y = torch.empty_like(x)
    mean, rstd = torch.empty(N, device="cuda"), torch.empty(N, device="cuda")
    bs.bsmm_layer_norm(x, g, b, y, mean, rstd, 1, 1e-6, False)
    torch.cuda.synchronize()
    ry, _, _ = oln.layer_norm(synth.to_bits(P.x), P.g.numpy(), P.b.numpy(), 1, 1e-6, False, dtype)
    assert_close(y, ry, dtype, "y")


def test_layer_norm_empty():
    """N = 0: no output; the gradient's dg and db are zero."""
    C = 40
    x = torch.empty(0, C, device="cuda", dtype=torch.bfloat16)
    g, b = torch.ones(C, device="cuda"), torch.zeros(C, device="cuda")
    dg, db = torch.full((C,), 7.0, device="cuda"), torch.full((C,), 7.0, device="cuda")
    bs.bsmm_layer_norm(x, g, b, torch.empty_like(x), None, None, 1, 1e-6, False)
    bs.bsmm_layer_norm_grad(x, x, g, b, torch.empty(0, device="cuda"), torch.empty(0, device="cuda"),
                            torch.empty_like(x), dg, db, 1, False)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dg) == 0 and torch.count_nonzero(db) == 0


def test_layer_norm_autograd_and_determinism():
    N, C = 33, 4096
    print(f"case layer_norm autograd N={N} C={C}", flush=True)
    P = synth.norm_problem(np.random.default_rng(12), N, C, 1, "bf16")
    x = dev(P.x).requires_grad_(True)
    g = dev(P.g).requires_grad_(True)
    b = dev(P.b).requires_grad_(True)
    y = bs.layer_norm(x, g, b, axis=1, epsilon=1e-6, relu=False)
    y.backward(dev(P.dy))
    torch.cuda.synchronize()
    rdx, rdg, rdb = oln.layer_norm_grad(synth.to_bits(P.dy), synth.to_bits(P.x), P.g.numpy(), P.b.numpy(), 1,
                                        1e-6, False, "bf16")
    assert_close(x.grad, rdx, "bf16", "dx")
    assert rel_err(g.grad, rdg) <= 1e-5 and rel_err(b.grad, rdb) <= 1e-5
    y2 = bs.layer_norm(x.detach(), g.detach(), b.detach(), axis=1)
    assert torch.equal(y.detach(), y2)   # fixed summation order


@pytest.mark.parametrize("axis", [1, 0])
def test_layer_norm_full_size(axis):
    """The band workload's activation: N = 4096 vectors of C = 8192 bf16 features."""
    _run(4096, 8192, axis, "bf16", False, 99 + axis)
