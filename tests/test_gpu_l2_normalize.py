"""GPU parity of BlocksparseMatMul.l2_normalize (weight normalisation per output
feature) and its gradient against the float64 oracle, through the C ABI: block sizes
8/16/32, fp32/bf16/f16 weights and outputs, with and without a gain, C != K layouts
with empty block columns, an all-zero column (epsilon branch), autograd, and the
4096-wide Bernoulli(0.5) layout of the benchmark."""
import numpy as np
import pytest
import torch

import block_sparse_matrix_amd as bs
import synth
from gpu_util import TOL, TORCH_DT, assert_close, dev, rel_err
from oracle import l2_normalize as ol2

pytestmark = pytest.mark.gpu


def _layout(rng, R, S, p):
    L = (rng.random((R, S)) < p).astype(np.uint8)
    L[:, 1] = 0   # an empty block column
    L[:, -1] = 0  # and an empty last one (its list starts past the last entry)
    return L


@pytest.mark.parametrize("with_gain", [True, False])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("b", [8, 16, 32])
def test_l2_normalize(b, dtype, with_gain):
    print(f"case l2_normalize b={b} dtype={dtype} gain={with_gain}", flush=True)
    rng = np.random.default_rng(b * 10 + with_gain)
    L = _layout(rng, 7, 5, 0.5)
    m = bs.BlocksparseMatMul(L, block_size=b)
    P = synth.random_problem(rng, L, b, 1, 1, dtype, w_std=0.5)
    w = dev(P.w)
    g = torch.from_numpy((rng.random(m.K) + 0.5).astype(np.float32)) if with_gain else None
    out = torch.empty(w.shape, dtype=TORCH_DT[dtype], device="cuda")
    norms = torch.empty(m.K, device="cuda")
    bs.bsmm_l2_normalize(m.handle, w, None if g is None else dev(g), out, norms, 1e-6)
    dy = synth._draw(rng, tuple(w.shape), 1.0, dtype)
    dw = torch.empty(w.shape, device="cuda")
    dg = torch.empty(m.K, device="cuda") if with_gain else None
    bs.bsmm_l2_normalize_grad(m.handle, dev(dy), w, None if g is None else dev(g), dw, dg, 1e-6)
    torch.cuda.synchronize()
    wb = synth.to_bits(P.w)
    gn = None if g is None else g.numpy()
    rout, rn = ol2.l2_normalize(L, wb, b, gn, 1e-6, dtype)
    assert_close(out, rout, dtype, "l2_normalize out")
    assert rel_err(norms, rn) <= 1e-5
    rdw, rdg = ol2.l2_normalize_grad(L, synth.to_bits(dy), wb, b, gn, 1e-6, dtype, dtype)
    assert rel_err(dw, rdw) <= 1e-5, ("dw", rel_err(dw, rdw))
    if with_gain:
        assert rel_err(dg, rdg) <= 1e-5, ("dgain", rel_err(dg, rdg))


def test_l2_normalize_zero_column():
    """A block column whose weights are all zero: norm sqrt(epsilon), output zero."""
    L = np.array([[1, 1], [1, 0]], np.uint8)
    b = 16
    m = bs.BlocksparseMatMul(L, block_size=b)
    w = torch.randn(3, b, b)
    w[1] = 0   # block (0, 1): the only block of column 1
    out = torch.empty_like(w, device="cuda")
    norms = torch.empty(m.K, device="cuda")
    bs.bsmm_l2_normalize(m.handle, dev(w), None, out, norms, 1e-6)
    dy = torch.randn(3, b, b)
    dw = torch.empty(3, b, b, device="cuda")
    bs.bsmm_l2_normalize_grad(m.handle, dev(dy), dev(w), None, dw, None, 1e-6)
    torch.cuda.synchronize()
    rout, rn = ol2.l2_normalize(L, w.numpy(), b, None, 1e-6)
    rdw, _ = ol2.l2_normalize_grad(L, dy.numpy(), w.numpy(), b, None, 1e-6)
    assert torch.count_nonzero(out[1]) == 0
    assert rel_err(norms, rn) <= 1e-5
    assert rel_err(dw, rdw) <= 1e-5


def test_l2_normalize_autograd_and_benchmark_layout():
    P = synth.workload_problem("hidden4096_b32_n64", "bf16", N=1)
    m = bs.BlocksparseMatMul(P.layout, block_size=32)
    print(f"case l2_normalize autograd nnz={m.nnz}", flush=True)
    w = dev(P.w).requires_grad_(True)
    g = dev(torch.linspace(0.5, 2.0, m.K)).requires_grad_(True)
    out = m.l2_normalize(w, g, 1e-6, torch.bfloat16)
    dy = torch.randn(out.shape, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    out.backward(dev(dy))
    torch.cuda.synchronize()
    wb = synth.to_bits(P.w)
    rout, _ = ol2.l2_normalize(P.layout, wb, 32, g.detach().cpu().numpy(), 1e-6, "bf16")
    assert_close(out, rout, "bf16", "out")
    rdw, rdg = ol2.l2_normalize_grad(P.layout, synth.to_bits(dy), wb, 32, g.detach().cpu().numpy(), 1e-6,
                                     "bf16", "bf16")
    assert_close(w.grad, rdw, "bf16", "dw")   # dw returned in w's dtype
    assert rel_err(g.grad, rdg) <= 1e-5


@pytest.mark.parametrize("b,dtype", [(8, "bf16"), (8, "f32"), (16, "f16"), (32, "f32"), (32, "bf16")])
def test_l2_normalize_long_columns(b, dtype):
    """Columns longer than the blocks one round of loads holds (they read the rest
    again) and longer than the 1024 entries a list record keeps inline (the rest come
    from the column list), beside short and empty columns."""
    print(f"case l2_normalize long columns b={b} dtype={dtype}", flush=True)
    rng = np.random.default_rng(700 + b)
    R = 1100
    L = np.zeros((R, 4), np.uint8)
    L[:, 0] = 1                               # 1100 blocks
    L[:, 2] = rng.random(R) < 0.1             # ~110 blocks
    L[rng.choice(R, 3, replace=False), 3] = 1  # 3 blocks; column 1 stays empty
    m = bs.BlocksparseMatMul(L, block_size=b)
    P = synth.random_problem(rng, L, b, 1, 1, dtype, w_std=0.5)
    w = dev(P.w)
    g = torch.from_numpy((rng.random(m.K) + 0.5).astype(np.float32))
    out = torch.empty(w.shape, dtype=TORCH_DT[dtype], device="cuda")
    norms = torch.empty(m.K, device="cuda")
    bs.bsmm_l2_normalize(m.handle, w, dev(g), out, norms, 1e-6)
    dy = synth._draw(rng, tuple(w.shape), 1.0, dtype)
    dw = torch.empty(w.shape, device="cuda")
    dg = torch.empty(m.K, device="cuda")
    bs.bsmm_l2_normalize_grad(m.handle, dev(dy), w, dev(g), dw, dg, 1e-6)
    torch.cuda.synchronize()
    wb = synth.to_bits(P.w)
    rout, rn = ol2.l2_normalize(L, wb, b, g.numpy(), 1e-6, dtype)
    assert_close(out, rout, dtype, "l2_normalize out")
    assert rel_err(norms, rn) <= 1e-5
    rdw, rdg = ol2.l2_normalize_grad(L, synth.to_bits(dy), wb, b, g.numpy(), 1e-6, dtype, dtype)
    assert rel_err(dw, rdw) <= 1e-5, ("dw", rel_err(dw, rdw))
    assert rel_err(dg, rdg) <= 1e-5, ("dgain", rel_err(dg, rdg))
