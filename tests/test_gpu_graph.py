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


@pytest.mark.parametrize("G,acc", [(3, False), (2, True)])
def test_capture_split_weight_gradient(G, acc):
    """The dense-tile weight gradient with both splits (tile parts, and the blocks outside
    the tiles in contraction parts that later launches add to) captured with a fixed
    workspace: every replay, with eager work between, gives the eager result bit for bit
    (accumulating: the eager result of the same starting dW)."""
    print(f"case graph capture split updat G={G} acc={acc}", flush=True)
    rng = np.random.default_rng(17 + G)
    L = np.zeros((32, 48), dtype=np.uint8)
    L[:, :40] = rng.random((32, 40)) < 0.45   # 20 dense tiles: the tile kernel, split
    L[:, 40:] = rng.random((32, 8)) < 0.1     # blocks outside the tiles
    N = 512
    P = synth.random_problem(rng, L, 32, N, 1, "bf16", G=G, w_std=0.1)
    m = bs.BlocksparseMatMul(L, block_size=32, feature_axis=1)
    h = m.handle
    assert m.kernel_name("updat", N, torch.bfloat16, G) == "dense_tiles"
    assert len(bs.bsmm_debug_lut(h, 19)) > 0
    xs, dys = [dev(t) for t in P.xs], [dev(t) for t in P.dys]
    nb = bs.bsmm_workspace_size(h, 2, N, torch.bfloat16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dw0 = torch.randn(m.w_shape, generator=torch.Generator().manual_seed(2)).cuda()
    dw = dw0.clone()
    bs.bsmm_updat(h, xs, dys, dw, N, accumulate=acc, ws=ws)   # eager (also uploads the tables)
    torch.cuda.synchronize()
    ref = dw.clone()
    dw.copy_(dw0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bs.bsmm_updat(h, xs, dys, dw, N, accumulate=acc, ws=ws)
    for rep in range(3):
        dw.copy_(dw0)                    # eager work between replays
        ws.fill_(0xFF)                   # the parts are written before they are read
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw, ref), f"replay {rep} differs from the eager result"
