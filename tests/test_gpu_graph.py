"""HIP-graph capture of the passes through the C ABI.

A handle's layout tables reach a device on its first call there (an allocation and an
asynchronous copy), so that first call is refused while its stream is being captured;
once made, fprop, bprop and updat capture into a graph whose replays give the eager
results bit for bit (the kernels have a fixed summation order)."""
import numpy as np
import pytest
import torch

import block_sparse_matrix_amd as bs
import synth
from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("b,fa,dtype", [(32, 1, "bf16"), (16, 0, "f32")])
def test_capture_after_first_call(b, fa, dtype):
    print(f"case graph capture b={b} fa={fa} {dtype}", flush=True)
    rng = np.random.default_rng(3)
    L = (rng.random((6, 5)) < 0.5).astype(np.uint8)
    L[0, 0] = 1
    N = 96
    P = synth.random_problem(rng, L, b, N, fa, dtype, G=1, w_std=0.1)
    m = bs.BlocksparseMatMul(L, block_size=b, feature_axis=fa)
    h = m.handle
    x, dy, w = dev(P.xs[0]), dev(P.dys[0]), dev(P.w)
    y, dx = torch.empty_like(dev(P.dys[0])), torch.empty_like(x)
    dw = torch.empty(m.w_shape, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    # first call on this device inside a capture: refused, nothing enqueued
    g0 = torch.cuda.CUDAGraph()
    with pytest.raises(bs.BsmmError) as ei:
        with torch.cuda.graph(g0):
            bs.bsmm_fprop(h, x, w, y, N)
    assert "capture" in str(ei.value)
    torch.cuda.synchronize()

    # eager (uploads the tables), then capture the three passes
    bs.bsmm_fprop(h, x, w, y, N)
    bs.bsmm_bprop(h, dy, w, dx, N)
    bs.bsmm_updat(h, [x], [dy], dw, N)
    torch.cuda.synchronize()
    ref = [y.clone(), dx.clone(), dw.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bs.bsmm_fprop(h, x, w, y, N)
        bs.bsmm_bprop(h, dy, w, dx, N)
        bs.bsmm_updat(h, [x], [dy], dw, N)
    for rep in range(3):
        for t in (y, dx, dw):
            t.fill_(float("nan"))   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, r in zip((y, dx, dw), ref):
            assert torch.equal(got, r), f"replay {rep} differs from the eager result"
