"""libbsmm.so on the CPU: it loads, exports every declared symbol, and validates
its arguments before any HIP call (so every error path runs without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_matrix_amd as bs
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INVALID, UNSUPPORTED, ALIGN = 1, 2, 3


def declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"BSMM_API\s+[\w\s\*]+?\b(bsmm_\w+)\s*\(", text))
    return names


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert {"bsmm_create", "bsmm_fprop", "bsmm_bprop", "bsmm_updat", "bsmm_identity_init"} <= names
    L = bs.lib()
    for n in sorted(names):
        assert hasattr(L, n), n


def _create(layout, b=8, fa=1):
    L = np.ascontiguousarray(layout, dtype=np.uint8)
    h = ctypes.c_void_p()
    st = bs.lib().bsmm_create(ctypes.byref(h), L.ctypes.data_as(ctypes.c_void_p), L.shape[0], L.shape[1], b, fa)
    return st, h


@pytest.mark.parametrize("layout,b,fa", [
    (np.ones((2, 2)), 4, 1), (np.ones((2, 2)), 64, 1), (np.ones((2, 2)), 8, 2), (np.ones((2, 2)), 8, -1),
    (np.array([[0, 2], [1, 1]]), 8, 1),
])
def test_create_rejects(layout, b, fa):
    st, h = _create(layout, b, fa)
    assert st == INVALID and not h.value
    assert bs.lib().bsmm_last_error().decode()


def test_create_rejects_null_and_empty():
    h = ctypes.c_void_p()
    assert bs.lib().bsmm_create(ctypes.byref(h), None, 2, 2, 8, 1) == INVALID
    z = np.zeros(1, dtype=np.uint8)
    assert bs.lib().bsmm_create(ctypes.byref(h), z.ctypes.data_as(ctypes.c_void_p), 0, 1, 8, 1) == INVALID
    assert bs.lib().bsmm_create(None, z.ctypes.data_as(ctypes.c_void_p), 1, 1, 8, 1) == INVALID


def test_all_zero_layout_is_valid():
    m = bs.BlocksparseMatMul(np.zeros((3, 2)), block_size=16, feature_axis=0)
    assert m.w_shape == (0, 16, 16)
    assert m.i_shape(5) == (48, 5) and m.o_shape(5) == (32, 5)
    with pytest.raises(bs.BsmmError):
        m.block_coord(0)


def test_shapes_and_block_coord():
    rng = np.random.default_rng(0)
    L = (rng.random((5, 7)) < 0.4).astype(np.uint8)
    for fa in (0, 1):
        m = bs.BlocksparseMatMul(L, block_size=32, feature_axis=fa)
        assert m.w_shape == (int(L.sum()), 32, 32)
        assert m.i_shape(3) == ((3, 160) if fa else (160, 3))
        assert m.o_shape(3) == ((3, 224) if fa else (224, 3))
        for t, (c, k) in enumerate(zip(*np.nonzero(L))):
            assert m.block_coord(t) == (c, k)
    with pytest.raises(bs.BsmmError):
        m.block_coord(int(L.sum()))
    with pytest.raises(bs.BsmmError):
        m.block_coord(-1)


def test_call_validation_before_gpu():
    L = bs.lib()
    st, h = _create(np.ones((2, 3)), 8, 1)
    assert st == 0
    vp = ctypes.c_void_p
    good = vp(0x10000)
    odd = vp(0x10008)
    try:
        # bad dtype, negative N, NULL pointers, misalignment
        assert L.bsmm_fprop(h, good, good, good, 4, 7, None, 0, None) == INVALID
        assert L.bsmm_fprop(h, good, good, good, -1, 0, None, 0, None) == INVALID
        assert L.bsmm_fprop(h, None, good, good, 4, 0, None, 0, None) == INVALID
        assert L.bsmm_fprop(h, good, None, good, 4, 0, None, 0, None) == INVALID
        assert L.bsmm_bprop(h, good, good, None, 4, 1, None, 0, None) == INVALID
        assert L.bsmm_fprop(h, odd, good, good, 4, 0, None, 0, None) == ALIGN
        assert L.bsmm_bprop(h, good, odd, good, 4, 2, None, 0, None) == ALIGN
        assert L.bsmm_fprop(None, good, good, good, 4, 0, None, 0, None) == INVALID
        assert L.bsmm_fprop(h, good, good, good, 1 << 40, 0, None, 0, None) == UNSUPPORTED
        # one row past the largest input activation the kernels address (2 GiB - 64 KiB):
        # x has 16 bf16 features per row (67 106 817 rows are 2 147 418 144 bytes), dy 24
        # (44 737 878 rows)
        assert L.bsmm_fprop(h, good, good, good, 67106817, 1, None, 0, None) == UNSUPPORTED
        assert L.bsmm_bprop(h, good, good, good, 44737878, 1, None, 0, None) == UNSUPPORTED
        # N = 0 is a no-op for fprop / bprop, even with NULL pointers
        assert L.bsmm_fprop(h, None, None, None, 0, 0, None, 0, None) == 0
        assert L.bsmm_bprop(h, None, None, None, 0, 1, None, 0, None) == 0
        arr = (vp * 8)(*([0x10000] * 8))
        assert L.bsmm_updat(h, arr, arr, 0, good, 4, 0, 0, None, 0, None) == INVALID
        assert L.bsmm_updat(h, arr, arr, 9, good, 4, 0, 0, None, 0, None) == INVALID
        assert L.bsmm_updat(h, arr, arr, 1, good, 4, 0, 5, None, 0, None) == INVALID
        assert L.bsmm_updat(h, arr, arr, 1, None, 4, 0, 0, None, 0, None) == INVALID
        assert L.bsmm_updat(h, None, arr, 1, good, 4, 0, 0, None, 0, None) == INVALID
        bad = (vp * 2)(0x10000, 0x10004)
        assert L.bsmm_updat(h, bad, bad, 2, good, 4, 0, 0, None, 0, None) == ALIGN
        # the accumulating form validates the same way; with N = 0 it adds nothing
        acc = L.bsmm_updat_accumulate
        assert acc(h, arr, arr, 0, good, 4, 0, 0, None, 0, None) == INVALID
        assert acc(h, arr, arr, 9, good, 4, 0, 0, None, 0, None) == INVALID
        assert acc(h, arr, arr, 1, good, 4, 0, 5, None, 0, None) == INVALID
        assert acc(h, arr, arr, 1, None, 4, 0, 0, None, 0, None) == INVALID
        assert acc(h, arr, arr, 1, odd, 4, 0, 0, None, 0, None) == ALIGN
        assert acc(h, bad, bad, 2, good, 4, 0, 0, None, 0, None) == ALIGN
        assert acc(h, None, None, 1, good, 0, 0, 0, None, 0, None) == 0
        # the allocation-free form validates the same way before touching the device
        na = L.bsmm_updat_noalloc
        assert na(None, arr, arr, 1, good, 4, 0, 0, None) == INVALID
        assert na(h, arr, arr, 0, good, 4, 0, 0, None) == INVALID
        assert na(h, arr, arr, 1, good, 4, 7, 0, None) == INVALID
        assert na(h, arr, arr, 1, None, 4, 0, 0, None) == INVALID
        assert na(h, arr, arr, 1, odd, 4, 0, 0, None) == ALIGN
        assert na(h, bad, bad, 2, good, 4, 0, 0, None) == ALIGN
        assert L.bsmm_identity_init(h, None, 0, None) == INVALID
        assert L.bsmm_identity_init(h, odd, 0, None) == ALIGN
        assert L.bsmm_identity_init(h, good, 9, None) == INVALID
        sz = ctypes.c_size_t(123)
        assert L.bsmm_workspace_size(h, 0, 64, 0, ctypes.byref(sz)) == 0 and sz.value == 0
        assert L.bsmm_workspace_size(h, 9, 64, 0, ctypes.byref(sz)) == INVALID
        assert L.bsmm_last_error().decode()
        for s in range(6):
            assert L.bsmm_status_string(s).decode().startswith("BSMM_")
        assert L.bsmm_profile_end(None, None) == INVALID
    finally:
        L.bsmm_destroy(h)
    L.bsmm_destroy(None)


def test_no_cpu_path():
    import torch
    m = bs.BlocksparseMatMul(np.ones((1, 1)), block_size=8)
    x = torch.zeros(2, 8)
    w = torch.zeros(1, 8, 8)
    with pytest.raises(ValueError):
        m.fprop(x, w)


def test_binding_rejects_wrong_sizes_before_any_call():
    """The C ABI sees pointers only; the binding checks every tensor's size, storage type
    and device against the plan first, so a wrong-shaped buffer is a ValueError rather
    than an out-of-bounds device access."""
    import torch
    m = bs.BlocksparseMatMul(np.ones((2, 3)), block_size=8)   # C = 16, K = 24, 6 blocks
    N = 4
    x, dy = torch.zeros(N, 16), torch.zeros(N, 24)
    w, y = torch.zeros(6, 8, 8), torch.zeros(N, 24)
    with pytest.raises(ValueError, match="shape"):
        bs.bsmm_fprop(m.handle, x, torch.zeros(5, 8, 8), y, N)
    with pytest.raises(ValueError, match="shape"):
        bs.bsmm_fprop(m.handle, x, w, torch.zeros(N, 16), N)
    with pytest.raises(ValueError, match="shape"):
        bs.bsmm_bprop(m.handle, dy, w, torch.zeros(N + 1, 16), N)
    with pytest.raises(ValueError, match="expected"):
        bs.bsmm_fprop(m.handle, x, w.to(torch.bfloat16), y, N)
    with pytest.raises(ValueError, match="shape"):
        bs.bsmm_updat(m.handle, [x], [dy], torch.zeros(5, 8, 8), N)
    with pytest.raises(ValueError, match="shape"):
        bs.bsmm_updat(m.handle, [x], [torch.zeros(N, 16)], w, N)
    with pytest.raises(ValueError):
        bs.bsmm_updat(m.handle, [x], [dy], w.to(torch.int32), N)
    # the class method: a wrong-shaped gradient to accumulate into
    with pytest.raises(ValueError, match="shape"):
        m.updat([x], [dy], out=torch.zeros(6, 8, 4), accumulate=True)
    with pytest.raises(ValueError, match="shape"):
        m.updat([x], [dy], out=torch.zeros(6 * 64), accumulate=True)
    with pytest.raises(ValueError):
        m.updat([x], [dy], out=torch.zeros(6, 8, 8, dtype=torch.float64), accumulate=True)


def test_kernel_choice_names():
    import torch
    rng = np.random.default_rng(0)
    L = (rng.random((16, 16)) < 0.5).astype(np.uint8)
    m32 = bs.BlocksparseMatMul(L, block_size=32, feature_axis=1)
    m8 = bs.BlocksparseMatMul(L, block_size=8, feature_axis=0)
    assert m32.kernel_name("fprop", 64, torch.bfloat16) == "rows_n64"
    assert m32.kernel_name("bprop", 64, torch.float32) == "rows_n64"
    assert m32.kernel_name("fprop", 65, torch.float32) == "list_rows128"
    assert m8.kernel_name("fprop", 64, torch.float32) == "list_n64_8waves"   # the rows kernel is 32x32 only
    long_col = np.zeros((300, 2), dtype=np.uint8)
    long_col[:, 0] = 1   # a 300-entry column list: more than the rows kernel takes
    mlong = bs.BlocksparseMatMul(long_col, block_size=32)
    assert mlong.kernel_name("fprop", 64, torch.bfloat16) == "list_n64"
    assert mlong.kernel_name("bprop", 64, torch.bfloat16) == "rows_n64"
    assert bs.BlocksparseMatMul(L, block_size=32, feature_axis=0).kernel_name("fprop", 64, torch.bfloat16) == "list_n64"
    assert m32.kernel_name("fprop", 4096, torch.bfloat16) == "output_groups"
    assert m32.kernel_name("bprop", 4096, torch.float16) == "output_groups"
    assert m32.kernel_name("fprop", 4096, torch.float32) == "list_weight_stack"
    assert m8.kernel_name("fprop", 4096, torch.bfloat16) == "list_weight_stack"
    assert m8.kernel_name("fprop", 512, torch.bfloat16) == "list_rows128"
    assert m32.kernel_name("fprop", 0, torch.bfloat16) == "none"
    assert m32.kernel_name("updat", 64, torch.bfloat16) == "row_runs"
    assert m32.kernel_name("updat", 4096, torch.bfloat16, group=8) == "row_groups"   # 4 tiles only
    big = bs.BlocksparseMatMul((rng.random((128, 128)) < 0.5).astype(np.uint8), block_size=32)
    assert big.kernel_name("updat", 4096, torch.bfloat16) == "dense_tiles"
    assert big.kernel_name("updat", 4096, torch.float32) == "row_groups"
    assert big.kernel_name("updat", 64, torch.bfloat16) == "row_runs"
    assert big.kernel_name("updat", 64, torch.bfloat16, group=2) == "blocks_2perwave"
    assert big.kernel_name("updat", 65, torch.float32) == "blocks_2perwave"
    assert m8.kernel_name("updat", 4096, torch.bfloat16) == "small_tiles"
    assert m8.kernel_name("updat", 4100, torch.bfloat16) == "row_groups"   # not whole 8-column chunks
    assert m8.kernel_name("updat", 4096, torch.float32) == "row_groups"
    assert m32.kernel_name("identity", 0, torch.bfloat16) == "identity"
    # 256x256 layouts at N = 4096: the output groups take sparse layouts once there
    # are >= 512 workgroups and the groups are >= 17 % full
    band = synth.workload_problem("hidden8192_b32_n4096_g8", "bf16", N=8, G=1).layout   # 24 % full
    assert bs.BlocksparseMatMul(band, block_size=32).kernel_name("fprop", 4096, torch.bfloat16) == "output_groups"
    assert bs.BlocksparseMatMul(band, block_size=32).kernel_name("fprop", 1024, torch.bfloat16) == "list_rows128"
    sparse = (rng.random((256, 256)) < 0.03).astype(np.uint8)   # about 14 % full
    assert bs.BlocksparseMatMul(sparse, block_size=32).kernel_name("bprop", 4096, torch.bfloat16) == "list_weight_stack"
    with pytest.raises(bs.BsmmError):
        m32.kernel_name("updat", 64, torch.bfloat16, group=9)


def test_weight_gradient_workspace_size():
    """The dense-tile weight gradient's workspace, from the layout alone: the tiles'
    split partials (parts = clamp(256 / tiles, 1, 8), 64 blocks of 4 KiB each per tile
    and part), then 8 parts of every block outside the tiles -- the latter only when
    the tiles can take the tile kernel (tiles x parts >= 128); 16-bit activations of
    32x32 blocks only, and none for N = 0."""
    import torch
    rng = np.random.default_rng(4)

    def ws(L, N=512, dt=torch.bfloat16):
        return bs.bsmm_workspace_size(bs.BlocksparseMatMul(L, block_size=32).handle, 2, N, dt)

    def counts(L):
        m = bs.BlocksparseMatMul(L, block_size=32)
        return len(bs.bsmm_debug_lut(m.handle, 16)) // 4, len(bs.bsmm_debug_lut(m.handle, 19))

    L = np.zeros((32, 48), dtype=np.uint8)   # 20 dense tiles and a sparse tile column
    L[:, :40] = rng.random((32, 40)) < 0.45
    L[:, 40:] = rng.random((32, 8)) < 0.1
    nt, nr = counts(L)
    assert nt >= 16 and nr > 0
    p = min(8, 256 // nt)
    assert ws(L) == (p * nt * 64 + 8 * nr) * 4096
    assert ws(L, dt=torch.float16) == ws(L)
    assert ws(L, dt=torch.float32) == 0 and ws(L, N=0) == 0
    few = np.zeros((16, 16), dtype=np.uint8)   # 4 dense tiles: tiles x parts = 32 < 128
    few[:, :] = rng.random((16, 16)) < 0.5
    few[:8, 8:] = 0
    few[0, 15] = 1                             # one block outside the tiles
    nt, nr = counts(few)
    assert 0 < nt < 16 and nr > 0
    assert ws(few) == 8 * nt * 64 * 4096       # the tiles' parts only
    many = (rng.random((128, 128)) < 0.5).astype(np.uint8)
    nt, nr = counts(many)
    assert nt >= 256                           # unsplit tiles: the rest's parts only
    assert ws(many) == 8 * nr * 4096
    empty_rest = np.ones((16, 16), dtype=np.uint8)
    assert counts(empty_rest)[1] == 0 and ws(empty_rest) == 8 * 4 * 64 * 4096
    assert ws(np.zeros((8, 8), dtype=np.uint8)) == 0


def test_force_kernel():
    import torch
    rng = np.random.default_rng(1)
    m = bs.BlocksparseMatMul((rng.random((16, 16)) < 0.5).astype(np.uint8), block_size=32)
    m.force_kernel("updat", "dense_tiles")
    assert m.kernel_name("updat", 4096, torch.bfloat16) == "dense_tiles"
    m.force_kernel("fprop", "list_rows128")
    assert m.kernel_name("fprop", 4096, torch.bfloat16) == "list_rows128"
    assert m.kernel_name("bprop", 4096, torch.bfloat16) == "output_groups"   # per pass
    m.force_kernel("fprop", None)
    assert m.kernel_name("fprop", 4096, torch.bfloat16) == "output_groups"
    with pytest.raises(bs.BsmmError):
        m.force_kernel("fprop", "dense_tiles")   # an updat kernel
    with pytest.raises(bs.BsmmError):
        m.force_kernel("updat", "no_such_kernel")
    # a forced family that cannot serve the call: reported as "none", rejected at call time
    m.force_kernel("updat", "dense_tiles")
    assert m.kernel_name("updat", 4096, torch.float32) == "none"


def test_layer_norm_arguments():
    """Argument checks of the layer-norm entry points (all before any HIP call)."""
    L = bs.lib()
    sz = ctypes.c_size_t()
    assert L.bsmm_layer_norm_workspace_size(4096, 8192, 1, 0, 1, ctypes.byref(sz)) == 0 and sz.value == 0
    assert L.bsmm_layer_norm_workspace_size(4096, 8192, 1, 1, 1, ctypes.byref(sz)) == 0
    assert sz.value == 2 * 256 * 8192 * 4              # 256 runs of 16 rows: dg and db partials
    assert L.bsmm_layer_norm_workspace_size(100, 300, 0, 0, 0, ctypes.byref(sz)) == 0
    assert sz.value == 3 * 100 * 8                     # 3 chunks of 128 rows x (mean, M2) per column
    assert L.bsmm_layer_norm_workspace_size(100, 300, 0, 1, 0, ctypes.byref(sz)) == 0
    assert sz.value == 3 * 100 * 8 + 2 * 4 * 300 * 4  # + 4 column blocks of dg and db partials
    assert L.bsmm_layer_norm_workspace_size(8, 8, 2, 0, 1, ctypes.byref(sz)) == 1   # axis
    assert L.bsmm_layer_norm_workspace_size(-1, 8, 1, 0, 1, ctypes.byref(sz)) == 1
    assert L.bsmm_layer_norm_workspace_size(8, 8, 1, 0, 9, ctypes.byref(sz)) == 1   # dtype
    vp = ctypes.c_void_p
    A, B = vp(0x10000), vp(0x20000)   # never dereferenced: every call below fails its checks
    f = ctypes.c_float

    def ln(x, y, N, C, axis, eps=1e-6, dt=1, ws=None, nb=0, mean=None, rstd=None):
        return L.bsmm_layer_norm(x, A, B, y, mean, rstd, N, C, axis, f(eps), 0, dt, ws, nb, None)

    assert ln(None, B, 4, 8, 1) == 1                  # x NULL
    assert ln(vp(0x10008), B, 4, 8, 1) == 3           # x not 16-byte aligned
    assert ln(A, B, 4, 8, 1, eps=-1.0) == 1           # epsilon < 0
    assert ln(A, B, 4, 8, 1, mean=A) == 1             # mean without rstd
    assert ln(A, B, 4, 8, 3) == 1                     # axis
    assert ln(A, B, 100, 300, 0) == 1                 # axis 0 needs a workspace
    assert ln(A, B, 4, 16384, 1, dt=0) == 2           # fp32 rows above 8192 features
    assert ln(A, B, 0, 8, 1) == 0                     # N = 0: no-op
    assert L.bsmm_layer_norm_grad(A, A, A, B, A, B, None, A, B, 4, 8, 1, 0, 1, None, 0, None) == 1   # dx NULL
    assert L.bsmm_layer_norm_grad(A, A, A, B, A, B, A, None, B, 4, 8, 1, 0, 1, None, 0, None) == 1   # dg NULL
    assert L.bsmm_layer_norm_grad(A, A, A, B, A, B, A, A, B, 4, 8, 1, 0, 1, None, 0, None) == 1      # no workspace
