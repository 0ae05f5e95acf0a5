"""The named workloads (the five configurations plus a supplementary half-dense one) at full size, launched exactly as bench.py launches them,
checked against the oracle on sampled outputs (GPU; calls through the C ABI).

Sampling: fprop/bprop outputs for a few minibatch rows (the oracle runs on those
rows of the input, which is the same function restricted to them) and updat for a
few block ids over the full (grouped) minibatch.  The tiny workload is compared in
full."""
import numpy as np
import pytest
import torch

import block_sparse_matrix_amd as bs
import oracle
import synth
from gpu_util import assert_close, dev

pytestmark = pytest.mark.gpu

CASES = [(name, dt) for name in synth.WORKLOAD_ORDER for dt in synth.WORKLOADS[name].dtypes]


def _rows(t: torch.Tensor, fa: int, idx: np.ndarray) -> torch.Tensor:
    return (t[idx] if fa == 1 else t[:, idx]).contiguous()


@pytest.mark.parametrize("name,dtype", CASES, ids=[f"{n}-{d}" for n, d in CASES])
def test_workload(name, dtype):
    print(f"workload {name} {dtype}", flush=True)
    P = synth.workload_problem(name, dtype)
    fa, b, N = P.fa, P.block, P.N
    m = bs.BlocksparseMatMul(P.layout, block_size=b, feature_axis=fa)
    w = dev(P.w)
    xs = [dev(t) for t in P.xs]
    dys = [dev(t) for t in P.dys]
    y = m.fprop(xs[0], w)
    dx = m.bprop(dys[0], w)
    dw = m.updat(xs, dys)
    torch.cuda.synchronize()
    bits = synth.to_bits
    rng = np.random.default_rng(7)
    if N <= 64 and P.R * b <= 256:
        rows = np.arange(N)
    else:
        rows = np.unique(np.concatenate([rng.choice(N, 8, replace=False), [0, N - 1]]))
    xs_s = bits(_rows(P.xs[0], fa, rows))
    dys_s = bits(_rows(P.dys[0], fa, rows))
    ry = oracle.fprop(P.layout, b, fa, xs_s, bits(P.w), len(rows), dtype)
    rdx = oracle.bprop(P.layout, b, fa, dys_s, bits(P.w), len(rows), dtype)
    assert_close(_rows(y.cpu(), fa, rows), ry, dtype, "fprop")
    assert_close(_rows(dx.cpu(), fa, rows), rdx, dtype, "bprop")
    nnz = P.nnz
    ids = np.arange(nnz) if nnz <= 64 else np.unique(
        np.concatenate([rng.choice(nnz, 30, replace=False), [0, nnz - 1]]))
    rdw = oracle.updat(P.layout, b, fa, [bits(t) for t in P.xs], [bits(t) for t in P.dys], N, dtype, ids=ids)
    assert_close(dw[torch.from_numpy(ids).cuda()], rdw, dtype, "updat")


def test_accumulate_at_benchmark_size():
    """The accumulating weight gradient as bench.py times it (hidden 4096, block 32, N = 64,
    bf16, fp32 dW): dW0 + sum, on sampled block ids against the oracle."""
    P = synth.workload_problem("hidden4096_b32_n64", "bf16")
    m = bs.BlocksparseMatMul(P.layout, block_size=32, feature_axis=1)
    rng = np.random.default_rng(9)
    dw0 = torch.from_numpy(rng.standard_normal(m.w_shape).astype(np.float32))
    out = dev(dw0)
    m.updat([dev(t) for t in P.xs], [dev(t) for t in P.dys], out=out, accumulate=True)
    torch.cuda.synchronize()
    ids = np.unique(np.concatenate([rng.choice(P.nnz, 30, replace=False), [0, P.nnz - 1]]))
    bits = synth.to_bits
    ref = dw0.numpy()[ids].astype(np.float64) + oracle.updat(P.layout, 32, 1, [bits(t) for t in P.xs],
                                                             [bits(t) for t in P.dys], P.N, "bf16", ids=ids)
    assert_close(out[torch.from_numpy(ids).cuda()], ref, "bf16", "updat accumulate")
