"""BlocksparseConv on the GPU against the CPU oracle (calls through the C ABI): fprop,
the input gradient and the filter gradient for 1-D, 2-D and 3-D images, strides,
dilations, SAME / VALID / explicit padding, blocks that share channels and channels in
no block, fp32 / bf16 / f16 storage; autograd through BlocksparseConv.__call__."""
import numpy as np
import pytest
import torch

import block_sparse_matrix_amd as bs
import synth
from gpu_util import assert_close, dev
from oracle import conv as oc

pytestmark = pytest.mark.gpu

CASES = [
    # N, C, K, Bc, Bk, nblocks, TRS, DHW, strides, dilates, padding
    (3, 6, 5, 2, 3, 4, (3,), (9,), (1,), (1,), "SAME"),
    (2, 8, 8, 4, 4, 3, (3, 3), (7, 6), (2, 1), (1, 1), "SAME"),
    (2, 8, 6, 2, 2, 5, (2, 3), (8, 9), (1, 2), (2, 1), "VALID"),
    (4, 16, 16, 8, 8, 3, (3, 3), (5, 5), (1, 1), (1, 1), 1),
    (2, 6, 6, 3, 3, 2, (2, 3, 2), (4, 5, 6), (1, 2, 1), (1, 1, 2), "SAME"),
    (2, 64, 64, 32, 32, 3, (3, 3), (12, 12), (1, 1), (1, 1), "SAME"),
    (1, 9, 70, 3, 64, 2, (1, 1), (3, 4), (1, 1), (1, 1), "VALID"),
]


def _f64(t):
    return t.detach().cpu().double().numpy()


@pytest.mark.parametrize("case", CASES, ids=[f"{len(c[6])}d-{c[10]}-B{c[3]}x{c[4]}" for c in CASES])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_conv(case, dtype):
    N, C, K, Bc, Bk, nb, TRS, DHW, st, dl, pad = case
    print(f"case conv {case} {dtype}", flush=True)
    g = oc.geometry(TRS, DHW, st, dl, pad)
    MPQ = g[2][3 - len(DHW):]
    rng = np.random.default_rng(C * 13 + K + len(DHW))
    P = synth.conv_problem(rng, N, C, K, Bc, Bk, nb, TRS, DHW, MPQ, dtype)
    # channel C-1 / K-1 in every problem: the plan's channel counts are one past the largest index
    P.BCK[0] = (P.BCK[0][0][:-1] + (C - 1,) if C - 1 not in P.BCK[0][0] else P.BCK[0][0],
                P.BCK[0][1][:-1] + (K - 1,) if K - 1 not in P.BCK[0][1] else P.BCK[0][1])
    conv = bs.BlocksparseConv(P.BCK, TRS, DHW, strides=st, dilates=dl, padding=pad)
    assert conv.C == C and conv.K == K and conv.MPQ == MPQ
    bck = oc.split_bck(P.BCK)
    F, I, dO = dev(P.F), dev(P.I), dev(P.dO)
    O = conv.fprop(F, I)
    dI = conv.bprop(F, dO)
    dF = conv.updat(I, dO)
    torch.cuda.synchronize()
    Fr, Ir, dOr = _f64(P.F), _f64(P.I), _f64(P.dO)
    assert_close(O, oc.fprop(bck, Fr, Ir, K, g).reshape(O.shape), dtype, "conv fprop")
    assert_close(dI, oc.bprop(bck, Fr, dOr, C, g).reshape(dI.shape), dtype, "conv bprop")
    assert_close(dF, oc.updat(bck, Ir, dOr, g).reshape(dF.shape), "f32" if dtype == "f32" else dtype, "conv updat")
    # output channels in no block are zero, input channels in no block get zero gradient
    used_k = set(int(k) for blk in P.BCK for k in blk[1])
    used_c = set(int(c) for blk in P.BCK for c in blk[0])
    for k in range(K):
        if k not in used_k:
            assert torch.count_nonzero(O[:, k]) == 0
    for c in range(C):
        if c not in used_c:
            assert torch.count_nonzero(dI[:, c]) == 0


def test_autograd_and_determinism():
    rng = np.random.default_rng(3)
    TRS, DHW = (3, 3), (10, 9)
    g = oc.geometry(TRS, DHW)
    P = synth.conv_problem(rng, 3, 32, 32, 8, 8, 6, TRS, DHW, g[2][1:], "f32", contiguous_blocks=True)
    conv = bs.BlocksparseConv(P.BCK, TRS, DHW)
    F = dev(P.F).requires_grad_()
    I = dev(P.I).requires_grad_()
    O = conv(F, I)
    O.backward(dev(P.dO))
    bck = oc.split_bck(P.BCK)
    assert_close(F.grad, oc.updat(bck, _f64(P.I), _f64(P.dO), g).reshape(F.shape), "f32", "dF")
    assert_close(I.grad, oc.bprop(bck, _f64(P.F), _f64(P.dO), conv.C, g).reshape(I.shape), "f32", "dI")
    O2 = conv.fprop(F.detach(), I.detach())
    dF2 = conv.updat(I.detach(), dev(P.dO))
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(dF2, F.grad)


MFMA_CASES = [
    # N, C, K, Bc, Bk, nblocks, TRS, DHW, padding
    (2, 64, 64, 32, 32, 3, (3, 3), (12, 20), "SAME"),   # 3 of 4 cells: channels in no block
    (3, 96, 64, 32, 16, 10, (3, 3), (9, 33), "SAME"),   # Bk 16, ragged last column tile
    (2, 128, 128, 64, 64, 3, (3, 1), (7, 16), "VALID"),  # two 32-channel slabs, Bk 64
    (2, 64, 64, 32, 32, 4, (3, 3), (10, 10), 2),        # explicit padding
    (4, 32, 32, 32, 32, 1, (7,), (50,), "SAME"),        # 1-D
    (2, 64, 64, 32, 32, 4, (2, 2), (8, 8), "SAME"),     # even filter: the odd pad after
    (4, 32, 32, 32, 32, 1, (7,), (48,), "SAME"),        # 1-D, width a multiple of 8: shifts -3 .. 3
    (2, 64, 64, 32, 32, 3, (1, 5), (8, 24), "SAME"),    # width a multiple of 8: shifts -2 .. 2
    (2, 64, 32, 32, 16, 4, (3, 3), (8, 16), "SAME"),    # row-form filter gradient, 2 tiles of 16x16
]


@pytest.mark.parametrize("case", MFMA_CASES, ids=[f"{c[6]}-{c[7]}-{c[8]}-B{c[3]}x{c[4]}" for c in MFMA_CASES])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_conv_matrix_core(case, dtype):
    """The matrix-core path (channel blocks on a grid, stride 1, 16-bit) against the oracle."""
    N, C, K, Bc, Bk, nb, TRS, DHW, pad = case
    print(f"case conv mfma {case} {dtype}", flush=True)
    g = oc.geometry(TRS, DHW, padding=pad)
    MPQ = g[2][3 - len(DHW):]
    rng = np.random.default_rng(C + K + nb + len(DHW))
    P = synth.conv_problem(rng, N, C, K, Bc, Bk, nb, TRS, DHW, MPQ, dtype, contiguous_blocks=True)
    conv = bs.BlocksparseConv(P.BCK, TRS, DHW, padding=pad)
    tdt = synth.DTYPES[dtype]
    assert conv.kernel_name("fprop", tdt) == "matrix_core"
    pads = g[5]
    want_b = Bk % 32 == 0 and Bc in (16, 32, 64) and pads[1] <= g[0][1] - 1 and pads[2] <= g[0][2] - 1
    assert conv.kernel_name("bprop", tdt) == ("matrix_core" if want_b else "matrix_core_gather")
    bck = oc.split_bck(P.BCK)
    F, I, dO = dev(P.F), dev(P.I), dev(P.dO)
    assert conv.kernel_name("updat", tdt) == ("matrix_core" if Bc % 16 == 0 and Bk % 16 == 0 else "direct")
    O = conv.fprop(F, I)
    dI = conv.bprop(F, dO)
    dF = conv.updat(I, dO)
    torch.cuda.synchronize()
    Cn, Kn = conv.C, conv.K
    Fr, Ir, dOr = _f64(P.F), _f64(P.I), _f64(P.dO)
    assert_close(O, oc.fprop(bck, Fr, Ir, Kn, g).reshape(O.shape), dtype, "conv fprop (matrix cores)")
    assert_close(dI, oc.bprop(bck, Fr, dOr, Cn, g).reshape(dI.shape), dtype, "conv bprop")
    assert_close(dF, oc.updat(bck, Ir, dOr, g).reshape(dF.shape), dtype, "conv updat")
    dF2 = conv.updat(I, dO)
    torch.cuda.synchronize()
    assert torch.equal(dF, dF2)
    O2 = conv.fprop(F, I)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)


def test_conv_filter_gradient_split():
    """The matrix-core filter gradient with its contraction split over the images (fp32
    partials in the workspace, summed in part order) and without a workspace (one part),
    both against the oracle."""
    import ctypes
    N, C, B, TRS, DHW = 8, 32, 32, (3, 3), (32, 32)
    g = oc.geometry(TRS, DHW)
    rng = np.random.default_rng(77)
    P = synth.conv_problem(rng, N, C, C, B, B, 1, TRS, DHW, g[2][1:], "bf16", contiguous_blocks=True)
    conv = bs.BlocksparseConv(P.BCK, TRS, DHW)
    n = ctypes.c_size_t()
    assert bs.lib().bsmm_conv_workspace_size(conv.handle, N, 1, ctypes.byref(n)) == 0
    assert n.value == 8 * B * 9 * B * 4        # 8 parts
    I, dO = dev(P.I), dev(P.dO)
    dF = conv.updat(I, dO)
    dF1 = torch.empty_like(dF)
    bs.lib().bsmm_conv_updat(conv.handle, ctypes.c_void_p(I.data_ptr()), ctypes.c_void_p(dO.data_ptr()),
                             ctypes.c_void_p(dF1.data_ptr()), N, 1, None, 0,
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    ref = oc.updat(oc.split_bck(P.BCK), _f64(P.I), _f64(P.dO), g).reshape(dF.shape)
    assert_close(dF, ref, "bf16", "split filter gradient")
    assert_close(dF1, ref, "bf16", "unsplit filter gradient")
    assert torch.equal(dF, conv.updat(I, dO))   # deterministic


def test_bench_configuration_sampled_images():
    """The configuration bench.py times (C = K = 256 in 32x32-channel blocks, 32 of 64,
    3x3, 32x32 images, N = 32, SAME, bf16, the same seed), on the kernels it launches;
    fprop / input gradient checked on two images (each image's outputs depend on that
    image only), the filter gradient (a sum over all images) on three sampled blocks
    (each block's gradient depends on its own channel lists only)."""
    N, C, B, TRS, DHW = 32, 256, 32, (3, 3), (32, 32)
    nb = (C // B) * (C // B) // 2
    P = synth.conv_problem(np.random.default_rng(23), N, C, C, B, B, nb, TRS, DHW, DHW, "bf16",
                           contiguous_blocks=True)
    conv = bs.BlocksparseConv(P.BCK, TRS, DHW)
    for p in ("fprop", "bprop", "updat"):
        assert conv.kernel_name(p) == "matrix_core"
    F, I, dO = dev(P.F), dev(P.I), dev(P.dO)
    O = conv.fprop(F, I)
    dI = conv.bprop(F, dO)
    dF = conv.updat(I, dO)
    torch.cuda.synchronize()
    g = oc.geometry(TRS, DHW)
    bck = oc.split_bck(P.BCK)
    Fr = _f64(P.F)
    for n in (0, N - 1):
        Irn, dOn = _f64(P.I[n:n + 1]), _f64(P.dO[n:n + 1])
        assert_close(O[n:n + 1], oc.fprop(bck, Fr, Irn, conv.K, g).reshape(1, conv.K, *DHW), "bf16", "fprop")
        assert_close(dI[n:n + 1], oc.bprop(bck, Fr, dOn, conv.C, g).reshape(1, conv.C, *DHW), "bf16", "bprop")
    blocks = [0, nb // 2, nb - 1]
    sub = (bck[0][blocks], bck[1][blocks])
    ref = oc.updat(sub, _f64(P.I), _f64(P.dO), g).reshape((len(blocks),) + tuple(dF.shape[1:]))
    assert_close(dF[blocks], ref, "bf16", "updat")


@pytest.mark.parametrize("Bc,Bk,TRS,DHW,pad", [
    (16, 16, (3, 3), (8, 16), "SAME"),    # one 16x16 tile: 8 waves split each step
    (16, 32, (2, 1), (6, 8), "VALID"),    # two tiles, an even filter height
    (64, 16, (3, 3), (9, 8), 1),          # four tiles, explicit padding
    (64, 64, (1, 3), (4, 24), "SAME"),    # sixteen tiles: two per wave
])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_conv_filter_gradient_rows(Bc, Bk, TRS, DHW, pad, dtype):
    """The row-form matrix-core filter gradient (one workgroup per block and filter row,
    every column tap of the row) for every tile count a wave split can take, against the
    oracle; deterministic."""
    print(f"case conv rows Bc={Bc} Bk={Bk} {TRS} {DHW} {pad} {dtype}", flush=True)
    N, C, K = 3, 2 * Bc, 2 * Bk
    g = oc.geometry(TRS, DHW, padding=pad)
    MPQ = g[2][3 - len(DHW):]
    rng = np.random.default_rng(Bc * 7 + Bk + len(TRS))
    P = synth.conv_problem(rng, N, C, K, Bc, Bk, 3, TRS, DHW, MPQ, dtype, contiguous_blocks=True)
    conv = bs.BlocksparseConv(P.BCK, TRS, DHW, padding=pad)
    assert conv.kernel_name("updat", synth.DTYPES[dtype]) == "matrix_core"
    I, dO = dev(P.I), dev(P.dO)
    dF = conv.updat(I, dO)
    torch.cuda.synchronize()
    ref = oc.updat(oc.split_bck(P.BCK), _f64(P.I), _f64(P.dO), g).reshape(dF.shape)
    assert_close(dF, ref, dtype, "row-form filter gradient")
    assert torch.equal(dF, conv.updat(I, dO))


GATHER_CASES = [
    # N, C, K, Bc, Bk, nblocks, TRS, DHW, strides, dilates, padding
    (2, 64, 64, 32, 32, 3, (3, 3), (12, 11), (2, 2), (1, 1), "SAME"),            # strided
    (2, 64, 32, 32, 16, 3, (3, 3), (10, 10), (1, 1), (2, 2), "SAME"),            # dilated, Bk 16
    (2, 32, 64, 16, 32, 4, (2, 3, 3), (4, 6, 5), (1, 1, 1), (1, 1, 1), "SAME"),  # 3-D
    (1, 32, 32, 16, 16, 3, (3, 2, 3), (7, 6, 9), (2, 1, 2), (1, 2, 1), "VALID"),  # 3-D strided + dilated
    (3, 64, 128, 64, 64, 2, (5,), (40,), (3,), (1,), 2),                          # 1-D, stride 3, pads 2
    (2, 64, 64, 32, 32, 4, (3, 3), (9, 9), (1, 1), (1, 1), "SAME"),              # stride 1 (fp32 takes it)
    (1, 32, 32, 32, 32, 1, (3, 3), (19, 17), (1, 1), (2, 1), "SAME"),            # 323 positions: ragged tile
    (2, 96, 32, 48, 16, 3, (3, 3), (8, 8), (2, 1), (1, 1), "SAME"),              # 48 contraction channels
    (2, 32, 16, 16, 8, 2, (3, 3), (6, 6), (1, 2), (1, 1), "SAME"),               # bprop over 8 channels
]


@pytest.mark.parametrize("case", GATHER_CASES,
                         ids=[f"{len(c[7])}d-st{c[8]}-dl{c[9]}-{c[10]}-B{c[3]}x{c[4]}" for c in GATHER_CASES])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_conv_gather(case, dtype):
    """The gathering matrix-core fprop / input gradient (any geometry and dtype) against
    the oracle, for the passes whose output channels per block are 16, 32 or 64, and the
    gathering filter gradient (Bc and Bk of 16, 32 or 64) split over a workspace and
    unsplit; deterministic."""
    import ctypes
    N, C, K, Bc, Bk, nb, TRS, DHW, st, dl, pad = case
    print(f"case conv gather {case} {dtype}", flush=True)
    g = oc.geometry(TRS, DHW, st, dl, pad)
    MPQ = g[2][3 - len(DHW):]
    rng = np.random.default_rng(C + 3 * K + nb + 5 * len(DHW) + Bk)
    P = synth.conv_problem(rng, N, C, K, Bc, Bk, nb, TRS, DHW, MPQ, dtype, contiguous_blocks=True)
    conv = bs.BlocksparseConv(P.BCK, TRS, DHW, strides=st, dilates=dl, padding=pad)
    tdt = synth.DTYPES[dtype]
    vec = 4 if dtype == "f32" else 8
    plain = dtype != "f32" and all(v == 1 for v in st) and all(v == 1 for v in dl) and len(DHW) < 3
    for name, co, ok in (("fprop", Bk, True), ("bprop", Bc, Bk % vec == 0)):
        got = conv.kernel_name(name, tdt)
        if co in (16, 32, 64) and ok:
            assert got == "matrix_core_gather" or (plain and got == "matrix_core"), (name, got)
        else:
            assert got == "direct", (name, got)
    if not plain:
        assert "matrix_core_gather" in (conv.kernel_name("fprop", tdt), conv.kernel_name("bprop", tdt))
    bck = oc.split_bck(P.BCK)
    F, I, dO = dev(P.F), dev(P.I), dev(P.dO)
    O = conv.fprop(F, I)
    dI = conv.bprop(F, dO)
    torch.cuda.synchronize()
    Fr, Ir, dOr = _f64(P.F), _f64(P.I), _f64(P.dO)
    assert_close(O, oc.fprop(bck, Fr, Ir, conv.K, g).reshape(O.shape), dtype, "conv fprop (gather)")
    assert_close(dI, oc.bprop(bck, Fr, dOr, conv.C, g).reshape(dI.shape), dtype, "conv bprop (gather)")
    O2 = conv.fprop(F, I)
    dI2 = conv.bprop(F, dO)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(dI, dI2)
    # filter gradient
    got = conv.kernel_name("updat", tdt)
    if Bc in (16, 32, 64) and Bk in (16, 32, 64):
        assert got == "matrix_core_gather" or (plain and got == "matrix_core"), ("updat", got)
    else:
        assert got == "direct", ("updat", got)
    dF = conv.updat(I, dO)   # with the workspace the library asks for
    dF1 = torch.empty_like(dF)
    code = {"f32": 0, "bf16": 1, "f16": 2}[dtype]
    assert bs.lib().bsmm_conv_updat(conv.handle, ctypes.c_void_p(I.data_ptr()), ctypes.c_void_p(dO.data_ptr()),
                                    ctypes.c_void_p(dF1.data_ptr()), N, code, None, 0,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    ref = oc.updat(bck, Ir, dOr, g).reshape(dF.shape)
    tol = "f32" if dtype == "f32" else dtype
    assert_close(dF, ref, tol, "conv updat (gather, split)")
    assert_close(dF1, ref, tol, "conv updat (gather, one part)")
    assert torch.equal(dF, conv.updat(I, dO))


@pytest.mark.parametrize("dtype,st", [("f32", (1, 1)), ("bf16", (2, 2))])
def test_conv_gather_large_grid(dtype, st):
    """The gathering kernels at a grid of 512 or more workgroups, where they take
    256-position tiles (smaller grids take 64): 64 images of 32 x 32, checked against
    the oracle on the first and last image (each image's outputs depend on that image
    only)."""
    N, C, B, TRS, DHW = 64, 64, 32, (3, 3), (32, 32)
    print(f"case conv gather large grid {dtype} strides={st}", flush=True)
    g = oc.geometry(TRS, DHW, st)
    MPQ = g[2][1:]
    P = synth.conv_problem(np.random.default_rng(91), N, C, C, B, B, 4, TRS, DHW, MPQ, dtype,
                           contiguous_blocks=True)
    conv = bs.BlocksparseConv(P.BCK, TRS, DHW, strides=st)
    tdt = synth.DTYPES[dtype]
    assert conv.kernel_name("bprop", tdt) == "matrix_core_gather"
    F, I, dO = dev(P.F), dev(P.I), dev(P.dO)
    O = conv.fprop(F, I)
    dI = conv.bprop(F, dO)
    torch.cuda.synchronize()
    bck = oc.split_bck(P.BCK)
    Fr = _f64(P.F)
    for n in (0, N - 1):
        Irn, dOn = _f64(P.I[n:n + 1]), _f64(P.dO[n:n + 1])
        assert_close(O[n:n + 1], oc.fprop(bck, Fr, Irn, conv.K, g).reshape(1, conv.K, *MPQ), dtype, "fprop")
        assert_close(dI[n:n + 1], oc.bprop(bck, Fr, dOn, conv.C, g).reshape(1, conv.C, *DHW), dtype, "bprop")
