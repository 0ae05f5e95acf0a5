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
