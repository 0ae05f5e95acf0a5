"""HIP path against the CPU oracle, element by element (GPU; calls through the C ABI).

Small random problems cover every (block size, feature_axis, dtype, pass) at sizes
that span several tiles and end in a ragged minibatch tail; special cases cover
identity_init (bit-exact), empty rows/columns, an all-zero layout, all-ones = dense,
determinism, grouped weight gradients and low-precision dW."""
import numpy as np
import pytest
import torch

import block_sparse_matrix_amd as bs
import oracle
import synth
from gpu_util import TOL, TORCH_DT, assert_close, dev, rel_err

pytestmark = pytest.mark.gpu


def _prob(seed, R, S, b, N, fa, dtype, G=1, density=0.45):
    rng = np.random.default_rng(seed)
    L = (rng.random((R, S)) < density).astype(np.uint8)
    L[0, :] = 0          # an empty input block row -> dx zero there
    L[:, S - 1] = 0      # an empty output block column -> y zero there
    L[1, 0] = 1
    return synth.random_problem(rng, L, b, N, fa, dtype, G=G, w_std=0.1)


def _run_all(P, dtype):
    m = bs.BlocksparseMatMul(P.layout, block_size=P.block, feature_axis=P.fa)
    w = dev(P.w)
    xs = [dev(t) for t in P.xs]
    dys = [dev(t) for t in P.dys]
    y = m.fprop(xs[0], w)
    dx = m.bprop(dys[0], w)
    dw = m.updat(xs, dys)
    torch.cuda.synchronize()
    return y, dx, dw


def _oracle_all(P, dtype):
    bits = synth.to_bits
    y = oracle.fprop(P.layout, P.block, P.fa, bits(P.xs[0]), bits(P.w), P.N, dtype)
    dx = oracle.bprop(P.layout, P.block, P.fa, bits(P.dys[0]), bits(P.w), P.N, dtype)
    dw = oracle.updat(P.layout, P.block, P.fa, [bits(t) for t in P.xs], [bits(t) for t in P.dys], P.N, dtype)
    return y, dx, dw


@pytest.mark.parametrize("N", [37, 200])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fa", [1, 0])
@pytest.mark.parametrize("b", [32, 16, 8])
def test_matrix(b, fa, dtype, N):
    print(f"case b={b} fa={fa} dtype={dtype} N={N}", flush=True)
    P = _prob(1000 * b + 10 * fa + N, 5, 7, b, N, fa, dtype)
    y, dx, dw = _run_all(P, dtype)
    ry, rdx, rdw = _oracle_all(P, dtype)
    assert_close(y, ry, dtype, "fprop")
    assert_close(dx, rdx, dtype, "bprop")
    # dW is fp32: its only rounding is fp32 accumulation of exactly decoded products
    assert_close(dw, rdw, "f32" if dtype == "f32" else dtype, "updat")
    # structural zeros: empty column of the layout and empty row
    Kb = P.block
    ycols = y[:, -Kb:] if fa == 1 else y[-Kb:, :]
    dxrows = dx[:, :Kb] if fa == 1 else dx[:Kb, :]
    assert torch.count_nonzero(ycols) == 0 and torch.count_nonzero(dxrows) == 0


@pytest.mark.parametrize("N", [1, 3, 63, 64, 65, 129])
def test_ragged_minibatch(N):
    for b, fa, dtype in [(32, 1, "bf16"), (16, 0, "f16"), (8, 0, "bf16"), (8, 1, "f32")]:
        print(f"case N={N} b={b} fa={fa} dtype={dtype}", flush=True)
        P = _prob(N * 7 + b, 4, 3, b, N, fa, dtype, G=2)
        y, dx, dw = _run_all(P, dtype)
        ry, rdx, rdw = _oracle_all(P, dtype)
        assert_close(y, ry, dtype, "fprop")
        assert_close(dx, rdx, dtype, "bprop")
        assert_close(dw, rdw, dtype, "updat")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fa", [1, 0])
@pytest.mark.parametrize("b", [32, 16, 8])
def test_identity_init_bit_exact(b, fa, dtype):
    print(f"case identity b={b} fa={fa} dtype={dtype}", flush=True)
    rng = np.random.default_rng(b + fa)
    R = 6
    L = ((rng.random((R, R)) < 0.4) | np.eye(R, dtype=bool)).astype(np.uint8)
    m = bs.BlocksparseMatMul(L, block_size=b, feature_axis=fa)
    w = m.identity_init(gpu=True, dtype=TORCH_DT[dtype])
    ref = oracle.identity(L, b)
    assert np.array_equal(w.float().cpu().numpy(), ref.astype(np.float32))
    host = m.identity_init(gpu=False)
    assert np.array_equal(host, ref.astype(np.float32))
    N = 77
    x = dev(torch.randn(m.i_shape(N), generator=torch.Generator().manual_seed(1)).to(TORCH_DT[dtype]))
    y = m.fprop(x, w)
    dx = m.bprop(x, w)
    torch.cuda.synchronize()
    assert torch.equal(y, x) and torch.equal(dx, x)


def test_identity_partial_diagonal():
    L = np.array([[1, 1, 0], [0, 0, 1], [1, 0, 1]], dtype=np.uint8)   # (1,1) absent
    m = bs.BlocksparseMatMul(L, block_size=16, feature_axis=1)
    w = m.identity_init(gpu=True, dtype=torch.bfloat16)
    x = dev(torch.randn(20, 48).to(torch.bfloat16))
    y = m.fprop(x, w)
    torch.cuda.synchronize()
    assert torch.equal(y[:, :16], x[:, :16]) and torch.equal(y[:, 32:], x[:, 32:])
    assert torch.count_nonzero(y[:, 16:32]) == 0


@pytest.mark.parametrize("fa", [1, 0])
def test_all_zero_layout(fa):
    m = bs.BlocksparseMatMul(np.zeros((2, 3)), block_size=8, feature_axis=fa)
    x = dev(torch.randn(m.i_shape(10)))
    dy = dev(torch.randn(m.o_shape(10)))
    w = torch.empty(m.w_shape, device="cuda")
    y = torch.full(m.o_shape(10), 7.0, device="cuda")
    dx = torch.full(m.i_shape(10), 7.0, device="cuda")
    bs.bsmm_fprop(m.handle, x, w, y, 10)
    bs.bsmm_bprop(m.handle, dy, w, dx, 10)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0 and torch.count_nonzero(dx) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_ones_layout_is_dense(dtype):
    R, S, b, N = 4, 3, 32, 96
    rng = np.random.default_rng(5)
    P = synth.random_problem(rng, np.ones((R, S), np.uint8), b, N, 1, dtype, w_std=0.1)
    y, dx, dw = _run_all(P, dtype)
    Wd = P.w.double().reshape(R, S, b, b).permute(0, 2, 1, 3).reshape(R * b, S * b)
    X, DY = P.xs[0].double(), P.dys[0].double()
    assert_close(y, (X @ Wd).numpy(), dtype, "fprop")
    assert_close(dx, (DY @ Wd.T).numpy(), dtype, "bprop")
    full = (X.T @ DY).reshape(R, b, S, b).permute(0, 2, 1, 3).reshape(R * S, b, b)
    assert_close(dw, full.numpy(), dtype, "updat")


def test_deterministic():
    for b, fa, dtype in [(32, 1, "bf16"), (16, 0, "f16"), (8, 0, "f32")]:
        P = _prob(77 + b, 6, 6, b, 130, fa, dtype, G=3)
        a = _run_all(P, dtype)
        c = _run_all(P, dtype)
        for u, v in zip(a, c):
            iv = torch.int32 if u.dtype == torch.float32 else torch.int16
            assert torch.equal(u.view(iv), v.view(iv))


@pytest.mark.parametrize("G", [1, 2, 5, 8])
def test_grouped_updat(G):
    for b, fa, dtype in [(32, 1, "bf16"), (16, 0, "f16"), (8, 1, "f32")]:
        P = _prob(G * 31 + b, 3, 4, b, 40, fa, dtype, G=G)
        m = bs.BlocksparseMatMul(P.layout, block_size=b, feature_axis=fa)
        dw = bs.group_param_grads(m, [dev(t) for t in P.xs], [dev(t) for t in P.dys])
        ref = oracle.updat(P.layout, b, fa, [synth.to_bits(t) for t in P.xs],
                           [synth.to_bits(t) for t in P.dys], P.N, dtype)
        assert_close(dw, ref, dtype, f"grouped G={G}")


@pytest.mark.parametrize("dw_dtype", ["bf16", "f16"])
def test_low_precision_dw(dw_dtype):
    P = _prob(3, 3, 3, 16, 50, 1, "bf16")
    m = bs.BlocksparseMatMul(P.layout, block_size=16, feature_axis=1)
    dw = m.updat([dev(P.xs[0])], [dev(P.dys[0])], dw_dtype=TORCH_DT[dw_dtype])
    assert dw.dtype == TORCH_DT[dw_dtype]
    ref = oracle.updat(P.layout, 16, 1, [synth.to_bits(P.xs[0])], [synth.to_bits(P.dys[0])], 50, "bf16")
    assert_close(dw, ref, dw_dtype, "dW low precision")


def test_autograd():
    P = _prob(11, 4, 4, 32, 70, 1, "f32")
    m = bs.BlocksparseMatMul(P.layout, block_size=32, feature_axis=1)
    x = dev(P.xs[0]).requires_grad_()
    w = dev(P.w).requires_grad_()
    y = m(x, w)
    y.backward(dev(P.dys[0]))
    torch.cuda.synchronize()
    bits = synth.to_bits
    assert_close(x.grad, oracle.bprop(P.layout, 32, 1, bits(P.dys[0]), bits(P.w), 70), "f32", "dx")
    assert_close(w.grad, oracle.updat(P.layout, 32, 1, [bits(P.xs[0])], [bits(P.dys[0])], 70), "f32", "dw")


@pytest.mark.parametrize("N", [1, 5, 16, 17, 32, 33, 63, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_rows_small_minibatch(N, dtype):
    """The small-minibatch kernel (32x32 blocks, features last, N <= 64; one workgroup
    per list and 32-row minibatch tile): lists of 40 entries and of few, empty lists
    (zeros), every minibatch-tile count and ragged tail, bit-reproducible."""
    print(f"case rows N={N} dtype={dtype}", flush=True)
    rng = np.random.default_rng(500 + N)
    R = S = 40
    L = (rng.random((R, S)) < 0.3).astype(np.uint8)
    L[:, 0] = 1          # a 40-entry column list
    L[2, :] = 1          # a 40-entry row list
    L[:, 5] = 0          # an empty column: y zero there
    L[9, :] = 0          # an empty row: dx zero there
    P = synth.random_problem(rng, L, 32, N, 1, dtype, G=1, w_std=0.1)
    m = bs.BlocksparseMatMul(L, block_size=32, feature_axis=1)
    for p in ("fprop", "bprop"):
        assert m.kernel_name(p, N, TORCH_DT[dtype]) == "rows_n64"
    y, dx = m.fprop(dev(P.xs[0]), dev(P.w)), m.bprop(dev(P.dys[0]), dev(P.w))
    ry, rdx, _ = _oracle_all(P, dtype)
    assert_close(y, ry, dtype, "fprop")
    assert_close(dx, rdx, dtype, "bprop")
    assert torch.count_nonzero(y[:, 5 * 32:6 * 32]) == 0 and torch.count_nonzero(dx[:, 9 * 32:10 * 32]) == 0
    # bit-reproducible: a second run gives the same bits
    y2, dx2 = m.fprop(dev(P.xs[0]), dev(P.w)), m.bprop(dev(P.dys[0]), dev(P.w))
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(dx, dx2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rows_all_zero_layout(dtype):
    """No stored blocks: every list is empty and the small-minibatch kernel writes zeros."""
    L = np.zeros((3, 4), dtype=np.uint8)
    m = bs.BlocksparseMatMul(L, block_size=32, feature_axis=1)
    assert m.kernel_name("fprop", 40, TORCH_DT[dtype]) == "rows_n64"
    N = 40
    x = torch.randn(N, 96, device="cuda").to(TORCH_DT[dtype])
    dy = torch.randn(N, 128, device="cuda").to(TORCH_DT[dtype])
    w = torch.empty(0, 32, 32, dtype=TORCH_DT[dtype], device="cuda")
    y = torch.full((N, 128), 7.0, device="cuda").to(TORCH_DT[dtype])
    dx = torch.full((N, 96), 7.0, device="cuda").to(TORCH_DT[dtype])
    bs.bsmm_fprop(m.handle, x, w, y, N)
    bs.bsmm_bprop(m.handle, dy, w, dx, N)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0 and torch.count_nonzero(dx) == 0


@pytest.mark.parametrize("N", [512, 530, 2048, 2100])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fa", [1, 0])
@pytest.mark.parametrize("b", [32, 16, 8])
def test_long_minibatch(b, fa, dtype, N):
    """Minibatches that select the long-contraction kernels (grouped weight gradient,
    weights staged in LDS for N >= 2048), aligned and ragged."""
    print(f"case long b={b} fa={fa} dtype={dtype} N={N}", flush=True)
    P = _prob(7 * b + 3 * fa + N, 4, 5, b, N, fa, dtype, G=2 if N < 1000 else 1)
    y, dx, dw = _run_all(P, dtype)
    ry, rdx, rdw = _oracle_all(P, dtype)
    assert_close(y, ry, dtype, "fprop")
    assert_close(dx, rdx, dtype, "bprop")
    assert_close(dw, rdw, dtype, "updat")


@pytest.mark.parametrize("N", [64, 1000, 2048])
@pytest.mark.parametrize("b,fa,dtype", [(8, 1, "f32"), (8, 0, "bf16"), (8, 0, "f16"), (16, 1, "bf16"), (32, 0, "f16")])
def test_lists_longer_than_one_chunk(b, fa, dtype, N):
    """Block lists longer than one staged chunk: 1030 entries at N = 64 (the record
    holds the first 1024); at N = 1000, 300 entries (16-bit 8x8 blocks with features
    first stage 128 at a time, so the list walk takes three chunks, the last partial);
    at N = 2048 lists longer than the LDS weight stack holds (at most 187 entries of 8x8
    blocks, 18 of 32x32)."""
    R = 1030 if N == 64 else (300 if b < 32 else 40)
    print(f"case longlist b={b} fa={fa} dtype={dtype} N={N} R={R}", flush=True)
    rng = np.random.default_rng(11 * b + N)
    L = np.zeros((R, R), dtype=np.uint8)
    L[:, 1] = 1                       # one output block summing R inputs
    L[2, :] = 1                       # one input block feeding R outputs
    L[np.arange(R), np.arange(R)] = 1
    P = synth.random_problem(rng, L, b, N, fa, dtype, w_std=0.05)
    if N == 1000 and b == 8 and fa == 0:
        m = bs.BlocksparseMatMul(L, block_size=b, feature_axis=fa)
        for p in ("fprop", "bprop"):
            assert m.kernel_name(p, N, TORCH_DT[dtype]) == "list_rows128"
    y, dx, dw = _run_all(P, dtype)
    ry, rdx, rdw = _oracle_all(P, dtype)
    assert_close(y, ry, dtype, "fprop")
    assert_close(dx, rdx, dtype, "bprop")
    assert_close(dw, rdw, dtype, "updat")


@pytest.mark.parametrize("N", [1024, 1032, 1100, 2048])
@pytest.mark.parametrize("fa", [1, 0])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_output_groups(N, fa, dtype):
    """The output-group kernel (32x32 blocks, long minibatch): a ragged last tile, an
    output group with no block at all, a partial last group, an empty row and column."""
    if fa == 0 and N % 8:
        pytest.skip("features-first activations take the group kernel only for N % 8 == 0")
    print(f"case groups N={N} fa={fa} dtype={dtype}", flush=True)
    rng = np.random.default_rng(N + fa)
    L = (rng.random((12, 20)) < 0.5).astype(np.uint8)
    L[0, :] = 0
    L[:, 19] = 0
    L[:, 8:16] = 0
    L[3, 2] = 1
    P = synth.random_problem(rng, L, 32, N, fa, dtype, w_std=0.1)
    m = bs.BlocksparseMatMul(L, block_size=32, feature_axis=fa)
    for p in ("fprop", "bprop"):
        assert m.kernel_name(p, N, TORCH_DT[dtype]) == "output_groups"
    y, dx, dw = _run_all(P, dtype)
    ry, rdx, rdw = _oracle_all(P, dtype)
    assert_close(y, ry, dtype, "fprop")
    assert_close(dx, rdx, dtype, "bprop")
    assert_close(dw, rdw, dtype, "updat")
    Kb = 32
    ycols = y[:, 8 * Kb:16 * Kb] if fa == 1 else y[8 * Kb:16 * Kb, :]
    assert torch.count_nonzero(ycols) == 0


@pytest.mark.parametrize("N,G", [(512, 1), (520, 3), (1000, 2)])
@pytest.mark.parametrize("fa", [1, 0])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_updat_dense_tiles(N, G, fa, dtype):
    """Weight gradient by dense 8x8-block tiles plus row groups of the remaining blocks
    (32x32 blocks, long contraction): partial tiles at the layout's edges, a ragged
    minibatch, grouped steps."""
    if fa == 0 and N % 8:
        pytest.skip("features-first activations take the tile kernel only for N % 8 == 0")
    print(f"case tiles N={N} G={G} fa={fa} dtype={dtype}", flush=True)
    rng = np.random.default_rng(N + 10 * G + fa)
    R, S = 20, 27
    L = (rng.random((R, S)) < 0.12).astype(np.uint8)
    L[np.abs(np.subtract.outer(np.arange(R), np.arange(S))) <= 2] = 1
    L[16:20, 24:27] = 1
    P = synth.random_problem(rng, L, 32, N, fa, dtype, G=G, w_std=0.1)
    m = bs.BlocksparseMatMul(L, block_size=32, feature_axis=fa)
    # few tiles: the automatic choice prefers row groups, so the tile kernel is forced
    assert m.kernel_name("updat", N, TORCH_DT[dtype], G) == "row_groups"
    assert len(bs.bsmm_debug_lut(m.handle, 16)) > 0 and len(bs.bsmm_debug_lut(m.handle, 18)) > 0
    m.force_kernel("updat", "dense_tiles")
    assert m.kernel_name("updat", N, TORCH_DT[dtype], G) == "dense_tiles"
    dw = m.updat([dev(t) for t in P.xs], [dev(t) for t in P.dys])
    torch.cuda.synchronize()
    bits = synth.to_bits
    rdw = oracle.updat(P.layout, 32, fa, [bits(t) for t in P.xs], [bits(t) for t in P.dys], N, dtype)
    assert_close(dw, rdw, dtype, "updat")


@pytest.mark.parametrize("fa", [1, 0])
def test_updat_dense_tiles_unsplit(fa):
    """Enough dense tiles that the contraction is not split (no workspace), chosen
    automatically."""
    print(f"case tiles unsplit fa={fa}", flush=True)
    N = 512
    rng = np.random.default_rng(77 + fa)
    L = (rng.random((128, 128)) < 0.3).astype(np.uint8)
    P = synth.random_problem(rng, L, 32, N, fa, "bf16", w_std=0.1)
    m = bs.BlocksparseMatMul(L, block_size=32, feature_axis=fa)
    assert len(bs.bsmm_debug_lut(m.handle, 16)) // 4 >= 128
    # no tile partials; the blocks outside the tiles take their split parts
    nrest = len(bs.bsmm_debug_lut(m.handle, 19))
    assert nrest > 0
    assert bs.bsmm_workspace_size(m.handle, 2, N, torch.bfloat16) == 8 * nrest * 32 * 32 * 4
    assert m.kernel_name("updat", N, torch.bfloat16) == "dense_tiles"
    dw = m.updat([dev(t) for t in P.xs], [dev(t) for t in P.dys])
    torch.cuda.synchronize()
    bits = synth.to_bits
    rdw = oracle.updat(P.layout, 32, fa, [bits(t) for t in P.xs], [bits(t) for t in P.dys], N, "bf16")
    assert_close(dw, rdw, "bf16", "updat")


def _tiles_and_rest(rng):
    """20 dense 8x8-block tiles (Bernoulli(0.45) over 32 x 40 blocks) and a sparse last
    tile column (Bernoulli(0.1)), whose blocks stay outside the tiles."""
    L = np.zeros((32, 48), dtype=np.uint8)
    L[:, :40] = rng.random((32, 40)) < 0.45
    L[:, 40:] = rng.random((32, 8)) < 0.1
    return L


@pytest.mark.parametrize("fa,dtype,N,G,dw_dtype,acc", [
    (1, "bf16", 520, 3, "f32", False),   # per-step-group launches adding to the parts
    (1, "bf16", 1000, 1, "f32", False),  # one launch
    (0, "f16", 512, 2, "f32", False),
    (0, "bf16", 520, 1, "bf16", False),  # 16-bit gradient from the parts' fp32 sum
    (1, "f16", 512, 2, "f32", True),     # accumulating: the parts' sum added to dW
])
def test_updat_tiles_with_split_rest(fa, dtype, N, G, dw_dtype, acc):
    """Dense tiles with enough tiles for the split tile path, and blocks outside the tiles
    whose contraction is cut into eight parts (fp32 parts in the workspace after the
    tiles' partials, each part summed over the step groups, then the parts in order)."""
    if fa == 0 and N % 8:
        pytest.skip("features-first activations take the tile kernel only for N % 8 == 0")
    print(f"case tiles+rest fa={fa} {dtype} N={N} G={G} dw={dw_dtype} acc={acc}", flush=True)
    rng = np.random.default_rng(900 + N + G + fa)
    L = _tiles_and_rest(rng)
    m = bs.BlocksparseMatMul(L, block_size=32, feature_axis=fa)
    nt = len(bs.bsmm_debug_lut(m.handle, 16)) // 4
    nrest = len(bs.bsmm_debug_lut(m.handle, 19))
    assert nt >= 16 and nrest > 0
    split = min(8, 256 // nt)
    assert bs.bsmm_workspace_size(m.handle, 2, N, TORCH_DT[dtype]) == (split * nt * 64 + 8 * nrest) * 32 * 32 * 4
    assert m.kernel_name("updat", N, TORCH_DT[dtype], G) == "dense_tiles"
    P = synth.random_problem(rng, L, 32, N, fa, dtype, G=G, w_std=0.1)
    xs, dys = [dev(t) for t in P.xs], [dev(t) for t in P.dys]
    def run():
        if acc:
            out = dev(dw0)
        else:
            out = torch.full(m.w_shape, float("nan"), device="cuda").to(TORCH_DT[dw_dtype])
        bs.bsmm_updat(m.handle, xs, dys, out, N, accumulate=acc)
        torch.cuda.synchronize()
        return out

    bits = synth.to_bits
    if acc:
        dw0 = (torch.randn(m.w_shape, generator=torch.Generator().manual_seed(5)) * 3.0).to(TORCH_DT[dw_dtype])
        ref = oracle.updat_accumulate(L, 32, fa, bits(dw0), dw_dtype, [bits(t) for t in P.xs],
                                      [bits(t) for t in P.dys], N, dtype)
    else:
        ref = oracle.updat(L, 32, fa, [bits(t) for t in P.xs], [bits(t) for t in P.dys], N, dtype)
    dw = run()
    assert_close(dw, ref, dtype, "updat")
    assert torch.equal(dw, run())   # deterministic: a second call gives the same bits


@pytest.mark.parametrize("dw_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("b,fa,dtype,N,G,kind", [
    (32, 1, "bf16", 64, 1, None),            # row runs (one step group, N <= 64)
    (16, 0, "f16", 200, 2, None),
    (32, 1, "f32", 37, 1, None),
    (32, 1, "f32", 64, 1, "blocks_2perwave"),
    (32, 1, "f16", 20, 1, "row_runs"),
    (8, 0, "bf16", 1000, 1, "row_groups"),
    (8, 1, "f32", 600, 3, "row_groups"),
    (32, 0, "bf16", 520, 2, "dense_tiles"),  # split tiles: partials in the workspace, then their sum
    (32, 1, "f16", 1024, 1, "dense_tiles"),
])
def test_updat_accumulate(b, fa, dtype, N, G, kind, dw_dtype):
    """updat that adds into the stored gradient (dW += sum), for every weight-gradient
    kernel family and every gradient dtype, against the oracle's stored value plus sum."""
    print(f"case accumulate b={b} fa={fa} {dtype} N={N} G={G} {kind} dw={dw_dtype}", flush=True)
    rng = np.random.default_rng(b + N + G)
    L = (rng.random((16, 16) if b == 32 else (6, 9)) < 0.5).astype(np.uint8)
    L[0, 0] = 1
    P = synth.random_problem(rng, L, b, N, fa, dtype, G=G, w_std=0.1)
    m = bs.BlocksparseMatMul(L, block_size=b, feature_axis=fa)
    if kind:
        m.force_kernel("updat", kind)
        assert m.kernel_name("updat", N, TORCH_DT[dtype], G) == kind
    dw0 = (torch.randn(m.w_shape) * 3.0).to(TORCH_DT[dw_dtype])
    out = dev(dw0)
    m.updat([dev(t) for t in P.xs], [dev(t) for t in P.dys], out=out, accumulate=True)
    torch.cuda.synchronize()
    bits = synth.to_bits
    ref = oracle.updat_accumulate(L, b, fa, bits(dw0), dw_dtype, [bits(t) for t in P.xs],
                                  [bits(t) for t in P.dys], N, dtype)
    assert_close(out, ref, "f32" if dw_dtype == "f32" and dtype == "f32" else "bf16", "updat accumulate")
    # N = 0 adds nothing
    before = out.clone()
    m.updat([dev(t[:0] if fa == 1 else t[:, :0]) for t in P.xs],
            [dev(t[:0] if fa == 1 else t[:, :0]) for t in P.dys], out=out, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(out, before)


@pytest.mark.parametrize("N", [1, 16, 33, 64])
@pytest.mark.parametrize("dtype,dw_dtype", [("f32", "f32"), ("bf16", "f32"), ("f16", "f32"), ("f32", "bf16"),
                                            ("bf16", "f16")])
def test_updat_row_runs(N, dtype, dw_dtype):
    """The short-contraction weight gradient (32x32 blocks, features last, one step group
    of N <= 64 rows): row groups of up to 8 blocks, a row group that is a whole row's
    single block, empty rows; every gradient dtype; bit-reproducible."""
    print(f"case row_runs N={N} {dtype} dw={dw_dtype}", flush=True)
    rng = np.random.default_rng(900 + N)
    L = (rng.random((20, 24)) < 0.4).astype(np.uint8)
    L[3, :] = 1          # a 24-block row: three full row groups
    L[5, :] = 0
    L[5, 7] = 1          # a row of one block
    L[8, :] = 0          # an empty row
    P = synth.random_problem(rng, L, 32, N, 1, dtype, G=1, w_std=0.1)
    m = bs.BlocksparseMatMul(L, block_size=32, feature_axis=1)
    assert m.kernel_name("updat", N, TORCH_DT[dtype]) == "row_runs"
    xs, dys = [dev(P.xs[0])], [dev(P.dys[0])]
    dw = m.updat(xs, dys, dw_dtype=TORCH_DT[dw_dtype])
    dw2 = m.updat(xs, dys, dw_dtype=TORCH_DT[dw_dtype])
    torch.cuda.synchronize()
    bits = synth.to_bits
    ref = oracle.updat(L, 32, 1, [bits(P.xs[0])], [bits(P.dys[0])], N, dtype)
    assert_close(dw, ref, "f32" if dtype == "f32" and dw_dtype == "f32" else "bf16", "updat row_runs")
    assert torch.equal(dw, dw2)


@pytest.mark.parametrize("b,R,S,density", [(8, 40, 36, 0.1), (16, 20, 18, 0.3), (8, 64, 64, 1.0)])
@pytest.mark.parametrize("N,G,dtype,dw_dtype", [(256, 1, "bf16", "f32"), (264, 3, "f16", "f32"),
                                                (512, 1, "f16", "bf16"), (1024, 1, "bf16", "f32")])
def test_updat_small_tiles(b, R, S, density, N, G, dtype, dw_dtype):
    """The small-block weight-gradient tiles (8x8 / 16x16 blocks, features first): tiles
    of 256 x 256 features with partial edge tiles, an empty tile row, grouped steps,
    ragged last step, a full layout; every block against the oracle; then the
    accumulating form; bit-reproducible."""
    print(f"case small_tiles b={b} R={R} S={S} p={density} N={N} G={G} {dtype} dw={dw_dtype}", flush=True)
    rng = np.random.default_rng(b * 7 + N + G)
    L = (rng.random((R, S)) < density).astype(np.uint8)
    if density < 1.0:
        L[: 256 // b, S - 1] = 0   # a column that is empty in the first tile row
        L[0, 0] = 1
    P = synth.random_problem(rng, L, b, N, 0, dtype, G=G, w_std=0.1)
    m = bs.BlocksparseMatMul(L, block_size=b, feature_axis=0)
    assert m.kernel_name("updat", N, TORCH_DT[dtype], G) == "small_tiles"
    xs, dys = [dev(t) for t in P.xs], [dev(t) for t in P.dys]
    dw = m.updat(xs, dys, dw_dtype=TORCH_DT[dw_dtype])
    dw2 = m.updat(xs, dys, dw_dtype=TORCH_DT[dw_dtype])
    torch.cuda.synchronize()
    bits = synth.to_bits
    ref = oracle.updat(L, b, 0, [bits(t) for t in P.xs], [bits(t) for t in P.dys], N, dtype)
    assert_close(dw, ref, "f32" if dw_dtype == "f32" else "bf16", "updat small_tiles")
    assert torch.equal(dw, dw2)
    dw0 = (torch.randn(m.w_shape) * 3.0).to(TORCH_DT[dw_dtype])
    out = dev(dw0)
    m.updat(xs, dys, out=out, accumulate=True)
    torch.cuda.synchronize()
    refa = oracle.updat_accumulate(L, b, 0, bits(dw0), dw_dtype, [bits(t) for t in P.xs], [bits(t) for t in P.dys],
                                   N, dtype)
    assert_close(out, refa, "bf16", "updat small_tiles accumulate")


@pytest.mark.parametrize("group_size", [8, 4])
def test_group_param_grads_longer_than_a_group(group_size):
    """11 steps sharing one weight: the first group's launch writes the gradient, the
    later ones add into it; equal to the oracle's sum over all 11 steps."""
    rng = np.random.default_rng(group_size)
    L = (rng.random((5, 7)) < 0.5).astype(np.uint8)
    L[0, 0] = 1
    P = synth.random_problem(rng, L, 16, 96, 1, "bf16", G=11, w_std=0.1)
    m = bs.BlocksparseMatMul(L, block_size=16, feature_axis=1)
    dw = bs.group_param_grads(m, [dev(t) for t in P.xs], [dev(t) for t in P.dys], group_size=group_size)
    torch.cuda.synchronize()
    bits = synth.to_bits
    ref = oracle.updat(L, 16, 1, [bits(t) for t in P.xs], [bits(t) for t in P.dys], 96, "bf16")
    assert_close(dw, ref, "bf16", "grouped dW over 11 steps")
