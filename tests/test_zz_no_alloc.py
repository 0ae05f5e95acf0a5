"""The allocation-free weight gradient (bsmm_updat_noalloc) against bsmm_updat, through
the C ABI: the same kernels with the library's fixed scratch in place of the caller's
workspace, so the results must be identical bit for bit (and within the tolerance of
the oracle).  Two calls in a row on one handle, the second with a smaller minibatch and
fewer steps, on a layout whose dense weight-gradient tiles take the split path (the
scratch is used), and on one that needs no scratch at all."""
import numpy as np
import pytest
import torch

import block_sparse_matrix_amd as bs
import oracle
import synth
from gpu_util import assert_close, dev

pytestmark = pytest.mark.gpu


def _band(R, width):
    c = np.arange(R)
    return (np.abs(c[:, None] - c[None, :]) <= width).astype(np.uint8)


def _tiles_and_rest(rng):
    """20 dense 8x8-block tiles and a sparse last tile column outside them: the blocks
    outside the tiles take the split path too (their parts after the tiles' in the
    scratch)."""
    L = np.zeros((32, 48), dtype=np.uint8)
    L[:, :40] = rng.random((32, 40)) < 0.45
    L[:, 40:] = rng.random((32, 8)) < 0.1
    return L


@pytest.mark.parametrize("b,fa,dtype,layout", [(32, 1, "bf16", "band"), (32, 0, "f16", "band"),
                                                (32, 1, "bf16", "tiles_rest"), (16, 0, "f16", "random")])
def test_noalloc_matches_updat(b, fa, dtype, layout):
    rng = np.random.default_rng(77 + b + fa)
    if layout == "band":
        L = _band(64, 2)
    elif layout == "tiles_rest":
        L = _tiles_and_rest(rng)
    else:
        L = (rng.random((24, 20)) < 0.3).astype(np.uint8)
    m = bs.BlocksparseMatMul(L, block_size=b, feature_axis=fa)
    h = m.handle
    for call, (N, G) in enumerate([(512, 2), (256, 2)]):   # second call: a smaller input
        print(f"case noalloc b={b} fa={fa} {dtype} {layout} call={call} N={N} G={G}", flush=True)
        P = synth.random_problem(rng, L, b, N, fa, dtype, G=G, w_std=0.1)
        xs = [dev(t) for t in P.xs]
        dys = [dev(t) for t in P.dys]
        need = bs.bsmm_workspace_size(h, 2, N, xs[0].dtype)
        if layout != "random":
            assert need > 0, "this layout must take the split tile path"
        ref = torch.empty(m.w_shape, dtype=torch.float32, device="cuda")
        bs.bsmm_updat(h, xs, dys, ref, N)                  # also uploads the layout tables
        got = torch.full(m.w_shape, float("nan"), device="cuda")
        bs.bsmm_updat_noalloc(h, xs, dys, got, N)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "the allocation-free call differs from bsmm_updat"
        bits = synth.to_bits
        rdw = oracle.updat(L, b, fa, [bits(t) for t in P.xs], [bits(t) for t in P.dys], N, dtype)
        assert_close(got, rdw, dtype, "updat_noalloc")


def test_noalloc_needs_tables_on_the_device():
    """Before any other call on the device the tables are not there: the call refuses
    (it would have to allocate) and leaves dW untouched."""
    L = _band(16, 1)
    m = bs.BlocksparseMatMul(L, block_size=32, feature_axis=1)
    N = 64
    x = torch.randn(N, 512, device="cuda").to(torch.bfloat16)
    dy = torch.randn(N, 512, device="cuda").to(torch.bfloat16)
    dw = torch.full(m.w_shape, 3.0, device="cuda")
    with pytest.raises(bs.BsmmError) as ei:
        bs.bsmm_updat_noalloc(m.handle, [x], [dy], dw, N)
    assert "allocating entry point" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(dw == 3.0)


def test_noalloc_band_workload_size():
    """The band workload's weight gradient at its full size (hidden 8192, 32x32 blocks,
    N = 4096, 8 step groups): 32 tiles split 8 ways (64 MiB of parts) and 869 blocks
    outside them split 8 ways (27 MiB) fit the scratch; bit-identical to bsmm_updat with
    a caller workspace, on two calls in a row (the second with 2 step groups and N = 1024)."""
    wl = synth.WORKLOADS["hidden8192_b32_n4096_g8"]
    rng = np.random.default_rng(wl.seed)
    R = wl.hidden // wl.block
    L = synth.make_layout(wl.layout_kind, R, R, rng)
    m = bs.BlocksparseMatMul(L, block_size=32, feature_axis=1)
    h = m.handle
    gen = torch.Generator(device="cuda").manual_seed(5)
    for call, (N, G) in enumerate([(4096, 8), (1024, 2)]):
        print(f"case noalloc band workload call={call} N={N} G={G}", flush=True)
        xs = [(torch.randn(N, wl.hidden, device="cuda", generator=gen)).to(torch.bfloat16) for _ in range(G)]
        dys = [(torch.randn(N, wl.hidden, device="cuda", generator=gen)).to(torch.bfloat16) for _ in range(G)]
        need = bs.bsmm_workspace_size(h, 2, N, torch.bfloat16)
        assert 64 << 20 < need <= 128 << 20 if call == 0 else need > 0
        assert m.kernel_name("updat", N, torch.bfloat16, G) == "dense_tiles"
        ref = torch.empty(m.w_shape, dtype=torch.float32, device="cuda")
        bs.bsmm_updat(h, xs, dys, ref, N)
        got = torch.full(m.w_shape, float("nan"), device="cuda")
        bs.bsmm_updat_noalloc(h, xs, dys, got, N)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "the allocation-free call differs from bsmm_updat"
        del xs, dys
