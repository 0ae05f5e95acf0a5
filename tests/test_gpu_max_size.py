"""Input activations at the largest size the kernels read (2 GiB - 64 KiB: 32-bit
offsets), features last and features first, 32x32 and 8x8 blocks: fprop and bprop
against the oracle on sampled minibatch rows (fa 1) or columns (fa 0), each of which
depends on that row or column only, and the weight gradient (a sum over all 262 136
rows) on sampled blocks.  Inputs are drawn on the GPU from a seeded generator."""
import numpy as np
import pytest
import torch

import block_sparse_matrix_amd as bs
import oracle
import synth
from gpu_util import assert_close

pytestmark = pytest.mark.gpu

MAX_INPUT_BYTES = 0x7FFF0000   # 2 147 418 112


@pytest.mark.parametrize("b,fa,density", [(32, 1, 0.04), (8, 0, 0.01)])
def test_largest_inputs(b, fa, density):
    C = K = 4096
    N = MAX_INPUT_BYTES // (C * 2)   # 262 136 rows of 4096 bf16 values: exactly the limit
    assert N * C * 2 == MAX_INPUT_BYTES
    print(f"case max size b={b} fa={fa} N={N}", flush=True)
    rng = np.random.default_rng(40 + b)
    L = (rng.random((C // b, K // b)) < density).astype(np.uint8)
    L[0, 0] = L[-1, -1] = 1
    m = bs.BlocksparseMatMul(L, block_size=b, feature_axis=fa)
    gen = torch.Generator(device="cuda").manual_seed(11 + b)
    shape = (N, C) if fa == 1 else (C, N)
    x = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    dy = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    w = (torch.randn(m.w_shape, generator=gen, device="cuda") * 0.05).to(torch.bfloat16)
    assert x.numel() * 2 == MAX_INPUT_BYTES
    y = m.fprop(x, w)
    dx = m.bprop(dy, w)
    dw = m.updat([x], [dy])
    torch.cuda.synchronize()
    bits = synth.to_bits
    pick = np.unique(np.concatenate([rng.choice(N, 6, replace=False), [0, N - 1]]))
    sel = torch.from_numpy(pick).cuda()
    take = (lambda t: t[sel].cpu()) if fa == 1 else (lambda t: t[:, sel].cpu())
    wb = bits(w.cpu())
    ry = oracle.fprop(L, b, fa, bits(take(x)), wb, len(pick), "bf16")
    rdx = oracle.bprop(L, b, fa, bits(take(dy)), wb, len(pick), "bf16")
    assert_close(take(y), ry, "bf16", "fprop at the size limit")
    assert_close(take(dx), rdx, "bf16", "bprop at the size limit")
    del y, dx
    nnz = int(L.sum())
    ids = np.unique(np.concatenate([rng.choice(nnz, 4, replace=False), [0, nnz - 1]]))
    rdw = oracle.updat(L, b, fa, [bits(x.cpu())], [bits(dy.cpu())], N, "bf16", ids=ids)
    assert_close(dw[torch.from_numpy(ids).cuda()], rdw, "bf16", "updat at the size limit")
