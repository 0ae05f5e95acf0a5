"""Block-sparse matrix multiply for AMD MI355X, over the C ABI of libbsmm.so.

Python mirror of the BlocksparseMatMul interface in the kiteco/blocksparse README
("API Documentation" › blocksparse.matmul): a layout of zeros and ones, a block size
of 8, 16 or 32, the feature_axis choice of activation layout, the shape helpers,
block_coord, identity_init, __call__ with dw_dtype, and the grouped weight gradient
(group_param_grads becomes an explicit call, since PyTorch has no graph to rewrite).

This module only marshals arguments: every arithmetic step runs in libbsmm's HIP
kernels.  PyTorch supplies device memory and the current stream.  There is no CPU
path: tensors must live on a ROCm device, and a missing libbsmm.so raises.

The raw C entry points are exposed under their C names (bsmm_create, bsmm_fprop,
bsmm_bprop, bsmm_updat, bsmm_identity_init, ...) taking torch tensors.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "BlocksparseMatMul", "BsmmError", "group_param_grads", "lib", "LIB_PATH",
    "bsmm_create", "bsmm_destroy", "bsmm_fprop", "bsmm_bprop", "bsmm_updat", "bsmm_updat_accumulate",
    "bsmm_updat_noalloc",
    "bsmm_identity_init",
    "bsmm_w_shape", "bsmm_i_shape", "bsmm_o_shape", "bsmm_block_coord", "bsmm_workspace_size",
    "bsmm_debug_lut", "bsmm_profile_begin", "bsmm_profile_end", "bsmm_plan_info",
    "bsmm_layer_norm", "bsmm_layer_norm_grad", "bsmm_layer_norm_workspace_size", "layer_norm",
    "bsmm_l2_normalize", "bsmm_l2_normalize_grad",
    "SparseProj", "bsmm_proj_gather", "bsmm_proj_scatter", "bsmm_proj_scatter_add", "bsmm_proj_scatter_mul",
    "bsmm_proj_gather_mul", "BlocksparseConv", "bsmm_conv_fprop", "bsmm_conv_bprop", "bsmm_conv_updat",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsmm.so")

BSMM_OK = 0
DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
PASS = {"fprop": 0, "bprop": 1, "updat": 2, "identity": 3, "layer_norm": 4, "layer_norm_grad": 5,
        "l2_normalize": 6, "l2_normalize_grad": 7, "proj_gather": 8, "proj_scatter": 9, "proj_scatter_add": 10,
        "proj_scatter_mul": 11, "proj_gather_mul": 12, "conv_fprop": 13, "conv_bprop": 14, "conv_updat": 15}


class BsmmError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: status {status} ({msg})")
        self.status = status


_lib = None


def lib():
    """The loaded libbsmm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_matrix_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    P64 = ctypes.POINTER(i64)
    sz = ctypes.c_size_t
    sigs = {
        "bsmm_create": [ctypes.POINTER(vp), vp, i64, i64, i32, i32],
        "bsmm_w_shape": [vp, P64],
        "bsmm_i_shape": [vp, i64, P64],
        "bsmm_o_shape": [vp, i64, P64],
        "bsmm_block_coord": [vp, i64, P64, P64],
        "bsmm_plan_info": [vp, P64],
        "bsmm_workspace_size": [vp, i32, i64, i32, ctypes.POINTER(sz)],
        "bsmm_fprop": [vp, vp, vp, vp, i64, i32, vp, sz, vp],
        "bsmm_bprop": [vp, vp, vp, vp, i64, i32, vp, sz, vp],
        "bsmm_updat": [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, i64, i32, i32, vp, sz, vp],
        "bsmm_updat_accumulate": [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, i64, i32, i32, vp, sz, vp],
        "bsmm_updat_noalloc": [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, i64, i32, i32, vp],
        "bsmm_identity_init": [vp, vp, i32, vp],
        "bsmm_debug_lut": [vp, i32, P64, i64, P64],
        "bsmm_kernel_name": [vp, i32, i64, i32, i32, ctypes.POINTER(ctypes.c_char_p)],
        "bsmm_force_kernel": [vp, i32, ctypes.c_char_p],
        "bsmm_layer_norm_workspace_size": [i64, i64, i32, i32, i32, ctypes.POINTER(sz)],
        "bsmm_layer_norm": [vp, vp, vp, vp, vp, vp, i64, i64, i32, ctypes.c_float, i32, i32, vp, sz, vp],
        "bsmm_layer_norm_grad": [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, vp, sz, vp],
        "bsmm_l2_normalize": [vp, vp, vp, vp, vp, ctypes.c_float, i32, i32, vp],
        "bsmm_l2_normalize_grad": [vp, vp, vp, vp, vp, vp, ctypes.c_float, i32, i32, vp],
        "bsmm_proj_create": [ctypes.POINTER(vp), i64, i64, i64, i64, vp],
        "bsmm_conv_create": [ctypes.POINTER(vp), i64, i64, i64, vp, vp, i64, i64, vp, vp, vp, vp, i32, vp],
        "bsmm_conv_geometry": [vp, vp, vp],
        "bsmm_conv_kernel_name": [vp, i32, i32, ctypes.POINTER(ctypes.c_char_p)],
        "bsmm_conv_fprop": [vp, vp, vp, vp, i64, i32, vp],
        "bsmm_conv_bprop": [vp, vp, vp, vp, i64, i32, vp],
        "bsmm_conv_updat": [vp, vp, vp, vp, i64, i32, vp, sz, vp],
        "bsmm_conv_workspace_size": [vp, i64, i32, ctypes.POINTER(sz)],
        "bsmm_proj_info": [vp, P64, P64],
        "bsmm_proj_lut": [vp, vp, i64],
        "bsmm_proj_gather": [vp, vp, vp, i64, i32, i32, vp],
        "bsmm_proj_scatter": [vp, vp, vp, i64, i32, i32, vp],
        "bsmm_proj_scatter_add": [vp, vp, vp, vp, i64, i32, i32, vp],
        "bsmm_proj_scatter_mul": [vp, vp, vp, vp, i64, i32, i32, vp],
        "bsmm_proj_gather_mul": [vp, vp, vp, vp, i64, i32, i32, vp],
        "bsmm_profile_begin": [],
        "bsmm_profile_end": [ctypes.POINTER(ctypes.c_double), P64],
    }
    for name, args in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.bsmm_destroy.argtypes = [vp]
    L.bsmm_destroy.restype = None
    L.bsmm_proj_destroy.argtypes = [vp]
    L.bsmm_proj_destroy.restype = None
    L.bsmm_conv_destroy.argtypes = [vp]
    L.bsmm_conv_destroy.restype = None
    L.bsmm_status_string.argtypes = [ctypes.c_int]
    L.bsmm_status_string.restype = ctypes.c_char_p
    L.bsmm_last_error.argtypes = []
    L.bsmm_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int, func: str):
    if status != BSMM_OK:
        L = lib()
        raise BsmmError(status, func, f"{L.bsmm_status_string(status).decode()}: {L.bsmm_last_error().decode()}")


def _stream(t: Optional[torch.Tensor] = None):
    dev = t.device if t is not None else torch.device("cuda", torch.cuda.current_device())
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dev_ptr(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a ROCm device tensor (no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


# ---- raw C entry points, same names -------------------------------------------------
def bsmm_create(layout, block_size: int = 32, feature_axis: int = 1) -> ctypes.c_void_p:
    L = np.ascontiguousarray(np.asarray(layout), dtype=np.uint8) if not isinstance(layout, np.ndarray) \
        or layout.dtype != np.uint8 else np.ascontiguousarray(layout)
    if L.ndim != 2:
        raise ValueError("layout must be a 2-D array of zeros and ones")
    h = ctypes.c_void_p()
    _check(lib().bsmm_create(ctypes.byref(h), L.ctypes.data_as(ctypes.c_void_p), L.shape[0], L.shape[1],
                             int(block_size), int(feature_axis)), "bsmm_create")
    return h


def bsmm_destroy(h) -> None:
    lib().bsmm_destroy(h)


def bsmm_w_shape(h):
    out = (ctypes.c_int64 * 3)()
    _check(lib().bsmm_w_shape(h, out), "bsmm_w_shape")
    return tuple(out)


def bsmm_i_shape(h, N: int):
    out = (ctypes.c_int64 * 2)()
    _check(lib().bsmm_i_shape(h, N, out), "bsmm_i_shape")
    return tuple(out)


def bsmm_o_shape(h, N: int):
    out = (ctypes.c_int64 * 2)()
    _check(lib().bsmm_o_shape(h, N, out), "bsmm_o_shape")
    return tuple(out)


def bsmm_block_coord(h, block: int):
    c, k = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().bsmm_block_coord(h, block, ctypes.byref(c), ctypes.byref(k)), "bsmm_block_coord")
    return int(c.value), int(k.value)


def bsmm_plan_info(h):
    out = (ctypes.c_int64 * 5)()
    _check(lib().bsmm_plan_info(h, out), "bsmm_plan_info")
    return dict(zip(("R", "S", "block_size", "feature_axis", "nnz"), tuple(out)))


def bsmm_workspace_size(h, pass_: int, N: int, dtype: torch.dtype) -> int:
    out = ctypes.c_size_t()
    _check(lib().bsmm_workspace_size(h, pass_, N, DTYPE_CODE[dtype], ctypes.byref(out)), "bsmm_workspace_size")
    return int(out.value)


def bsmm_kernel_name(h, pass_: int, N: int, dtype: torch.dtype, group: int = 1) -> str:
    out = ctypes.c_char_p()
    _check(lib().bsmm_kernel_name(h, pass_, N, group, DTYPE_CODE[dtype], ctypes.byref(out)), "bsmm_kernel_name")
    return out.value.decode()


def bsmm_force_kernel(h, pass_: int, name: Optional[str]) -> None:
    _check(lib().bsmm_force_kernel(h, pass_, name.encode() if name else None), "bsmm_force_kernel")


def bsmm_debug_lut(h, which: int) -> np.ndarray:
    n = ctypes.c_int64()
    _check(lib().bsmm_debug_lut(h, which, None, 0, ctypes.byref(n)), "bsmm_debug_lut")
    out = np.zeros(max(n.value, 1), dtype=np.int64)
    _check(lib().bsmm_debug_lut(h, which, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n.value,
                                ctypes.byref(n)), "bsmm_debug_lut")
    return out[:n.value]


_STORAGE = (torch.float32, torch.bfloat16, torch.float16)


def _need(t: torch.Tensor, name: str, shape, dtype=None, device=None) -> None:
    """The library writes and reads exactly prod(shape) elements through t's pointer:
    reject a tensor of another size, storage type or device before any call."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.numel() != int(np.prod(shape)):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)} elements' worth")
    if t.dtype not in _STORAGE:
        raise ValueError(f"{name} must be float32, bfloat16 or float16, not {t.dtype}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} is {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _mm_check(h, a: torch.Tensor, w: torch.Tensor, out: torch.Tensor, N: int, names, bprop: bool) -> None:
    ishape, oshape = bsmm_i_shape(h, N), bsmm_o_shape(h, N)
    if bprop:
        ishape, oshape = oshape, ishape
    _need(a, names[0], ishape)
    _need(w, names[1], bsmm_w_shape(h), a.dtype, a.device)
    _need(out, names[2], oshape, a.dtype, a.device)


def _ws(h, pass_, N, dtype, device, ws: Optional[torch.Tensor] = None):
    """The pass's workspace: `ws` when given (at least bsmm_workspace_size bytes, reused
    across calls, e.g. by a captured graph), else a fresh allocation when one is needed."""
    nbytes = bsmm_workspace_size(h, pass_, N, dtype)
    if ws is not None:
        if ws.device != device or ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"ws must hold at least {nbytes} bytes on {device}")
        return ws, ws.numel() * ws.element_size()
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def bsmm_fprop(h, x: torch.Tensor, w: torch.Tensor, y: torch.Tensor, N: int,
               ws: Optional[torch.Tensor] = None) -> None:
    _mm_check(h, x, w, y, N, ("x", "w", "y"), False)
    ws, nb = _ws(h, 0, N, x.dtype, x.device, ws)
    _check(lib().bsmm_fprop(h, _dev_ptr(x, "x"), _dev_ptr(w, "w"), _dev_ptr(y, "y"), N, DTYPE_CODE[x.dtype],
                            _dev_ptr(ws, "ws"), nb, _stream(x)), "bsmm_fprop")


def bsmm_bprop(h, dy: torch.Tensor, w: torch.Tensor, dx: torch.Tensor, N: int,
               ws: Optional[torch.Tensor] = None) -> None:
    _mm_check(h, dy, w, dx, N, ("dy", "w", "dx"), True)
    ws, nb = _ws(h, 1, N, dy.dtype, dy.device, ws)
    _check(lib().bsmm_bprop(h, _dev_ptr(dy, "dy"), _dev_ptr(w, "w"), _dev_ptr(dx, "dx"), N,
                            DTYPE_CODE[dy.dtype], _dev_ptr(ws, "ws"), nb, _stream(dy)), "bsmm_bprop")


def bsmm_updat(h, xs: Sequence[torch.Tensor], dys: Sequence[torch.Tensor], dw: torch.Tensor, N: int,
               accumulate: bool = False, ws: Optional[torch.Tensor] = None) -> None:
    """dw = (or, with accumulate, dw +=) the sum over the steps of x_t^T . dy_t on the
    present blocks (bsmm_updat / bsmm_updat_accumulate)."""
    G = len(xs)
    if G != len(dys):
        raise ValueError("xs and dys differ in length")
    if not 1 <= G <= 8:
        raise ValueError("updat takes 1 to 8 (x, dy) pairs")
    ishape, oshape = bsmm_i_shape(h, N), bsmm_o_shape(h, N)
    for x, dy in zip(xs, dys):
        _need(x, "xs[t]", ishape, xs[0].dtype, xs[0].device)
        _need(dy, "dys[t]", oshape, xs[0].dtype, xs[0].device)
    _need(dw, "dw", bsmm_w_shape(h), None, xs[0].device)
    xp = (ctypes.c_void_p * max(G, 1))(*[_dev_ptr(t, "xs[t]").value for t in xs])
    dp = (ctypes.c_void_p * max(G, 1))(*[_dev_ptr(t, "dys[t]").value for t in dys])
    dt = xs[0].dtype if G else dw.dtype
    ws, nb = _ws(h, 2, N, dt, dw.device, ws)
    fn = "bsmm_updat_accumulate" if accumulate else "bsmm_updat"
    _check(getattr(lib(), fn)(h, xp, dp, G, _dev_ptr(dw, "dw"), N, DTYPE_CODE[dt], DTYPE_CODE[dw.dtype],
                              _dev_ptr(ws, "ws"), nb, _stream(dw)), fn)


def bsmm_updat_noalloc(h, xs: Sequence[torch.Tensor], dys: Sequence[torch.Tensor], dw: torch.Tensor,
                       N: int) -> None:
    """dw = the sum over the steps of x_t^T . dy_t (as bsmm_updat), with the library's fixed
    device scratch instead of a workspace: the call allocates nothing (bsmm_updat_noalloc)."""
    G = len(xs)
    if G != len(dys):
        raise ValueError("xs and dys differ in length")
    if not 1 <= G <= 8:
        raise ValueError("updat takes 1 to 8 (x, dy) pairs")
    ishape, oshape = bsmm_i_shape(h, N), bsmm_o_shape(h, N)
    for x, dy in zip(xs, dys):
        _need(x, "xs[t]", ishape, xs[0].dtype, xs[0].device)
        _need(dy, "dys[t]", oshape, xs[0].dtype, xs[0].device)
    _need(dw, "dw", bsmm_w_shape(h), None, xs[0].device)
    xp = (ctypes.c_void_p * G)(*[_dev_ptr(t, "xs[t]").value for t in xs])
    dp = (ctypes.c_void_p * G)(*[_dev_ptr(t, "dys[t]").value for t in dys])
    _check(lib().bsmm_updat_noalloc(h, xp, dp, G, _dev_ptr(dw, "dw"), N, DTYPE_CODE[xs[0].dtype],
                                    DTYPE_CODE[dw.dtype], _stream(dw)), "bsmm_updat_noalloc")


def bsmm_identity_init(h, w: torch.Tensor) -> None:
    _check(lib().bsmm_identity_init(h, _dev_ptr(w, "w"), DTYPE_CODE[w.dtype], _stream(w)), "bsmm_identity_init")


def bsmm_profile_begin() -> None:
    _check(lib().bsmm_profile_begin(), "bsmm_profile_begin")


def bsmm_profile_end():
    """Returns {pass: (total_ms, count)} of the kernel times recorded since begin."""
    ms = (ctypes.c_double * len(PASS))()
    cnt = (ctypes.c_int64 * len(PASS))()
    _check(lib().bsmm_profile_end(ms, cnt), "bsmm_profile_end")
    return {name: (ms[i], int(cnt[i])) for name, i in PASS.items()}


# ---- layer norm (README, "API Documentation" › blocksparse.norms › layer_norm) -----------
def bsmm_layer_norm_workspace_size(N: int, C: int, axis: int, grad: bool, dtype: torch.dtype) -> int:
    n = ctypes.c_size_t()
    _check(lib().bsmm_layer_norm_workspace_size(N, C, axis, int(bool(grad)), DTYPE_CODE[dtype], ctypes.byref(n)),
           "bsmm_layer_norm_workspace_size")
    return n.value


def _ln_dims(x: torch.Tensor, axis: int):
    if x.dim() != 2:
        raise ValueError("layer_norm takes a 2-D activation: (N, C) for axis=1, (C, N) for axis=0")
    if axis not in (0, 1):
        raise ValueError("axis must be 0 or 1")
    return (x.shape[0], x.shape[1]) if axis == 1 else (x.shape[1], x.shape[0])


def _ln_ws(N, C, axis, grad, dtype, device):
    nb = bsmm_layer_norm_workspace_size(N, C, axis, grad, dtype)
    return (torch.empty(nb, dtype=torch.uint8, device=device), nb) if nb else (None, 0)


def bsmm_layer_norm(x: torch.Tensor, g: torch.Tensor, b: torch.Tensor, y: torch.Tensor,
                    mean: Optional[torch.Tensor], rstd: Optional[torch.Tensor], axis: int = 1,
                    epsilon: float = 1e-6, relu: bool = False) -> None:
    N, C = _ln_dims(x, axis)
    ws, nb = _ln_ws(N, C, axis, False, x.dtype, x.device)
    _check(lib().bsmm_layer_norm(_dev_ptr(x, "x"), _dev_ptr(g, "g"), _dev_ptr(b, "b"), _dev_ptr(y, "y"),
                                 _dev_ptr(mean, "mean"), _dev_ptr(rstd, "rstd"), N, C, axis, float(epsilon),
                                 int(bool(relu)), DTYPE_CODE[x.dtype], _dev_ptr(ws, "ws"), nb, _stream(x)),
           "bsmm_layer_norm")


def bsmm_layer_norm_grad(dy: torch.Tensor, x: torch.Tensor, g: torch.Tensor, b: torch.Tensor,
                         mean: torch.Tensor, rstd: torch.Tensor, dx: torch.Tensor, dg: torch.Tensor,
                         db: torch.Tensor, axis: int = 1, relu: bool = False) -> None:
    N, C = _ln_dims(x, axis)
    ws, nb = _ln_ws(N, C, axis, True, x.dtype, x.device)
    _check(lib().bsmm_layer_norm_grad(_dev_ptr(dy, "dy"), _dev_ptr(x, "x"), _dev_ptr(g, "g"), _dev_ptr(b, "b"),
                                      _dev_ptr(mean, "mean"), _dev_ptr(rstd, "rstd"), _dev_ptr(dx, "dx"),
                                      _dev_ptr(dg, "dg"), _dev_ptr(db, "db"), N, C, axis, int(bool(relu)),
                                      DTYPE_CODE[x.dtype], _dev_ptr(ws, "ws"), nb, _stream(x)),
           "bsmm_layer_norm_grad")


def _ln_param(p: torch.Tensor, C: int, name: str) -> torch.Tensor:
    if p.dtype != torch.float32 or p.dim() != 1 or p.shape[0] != C:
        raise ValueError(f"{name} must be a float32 vector of the {C} features")
    return p


class _LayerNormFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, g, b, axis, epsilon, relu):
        N, C = _ln_dims(x, axis)
        _ln_param(g, C, "g")
        _ln_param(b, C, "b")
        y = torch.empty_like(x)
        mean = torch.empty(N, dtype=torch.float32, device=x.device)
        rstd = torch.empty(N, dtype=torch.float32, device=x.device)
        bsmm_layer_norm(x, g, b, y, mean, rstd, axis, epsilon, relu)
        ctx.save_for_backward(x, g, b, mean, rstd)
        ctx.axis, ctx.relu = axis, relu
        return y

    @staticmethod
    def backward(ctx, dy):
        x, g, b, mean, rstd = ctx.saved_tensors
        dx = torch.empty_like(x)
        dg = torch.empty_like(g)
        db = torch.empty_like(b)
        bsmm_layer_norm_grad(dy.contiguous(), x, g, b, mean, rstd, dx, dg, db, ctx.axis, ctx.relu)
        return dx, dg, db, None, None, None


def layer_norm(x: torch.Tensor, g: torch.Tensor, b: torch.Tensor, axis: int = 1, epsilon: float = 1e-6,
               relu: bool = False) -> torch.Tensor:
    """Layer norm over the feature axis of a block-sparse matmul activation, with the
    optional ReLU at the end (README, "API Documentation" › blocksparse.norms ›
    layer_norm).  axis=1: x is (N, C); axis=0: x is (C, N).  g, b: float32 (C,).
    Differentiable in x, g and b."""
    return _LayerNormFunction.apply(x, g, b, axis, epsilon, relu)


# ---- weight normalisation (README, BlocksparseMatMul.l2_normalize) --------------------
def bsmm_l2_normalize(h, w: torch.Tensor, gain: Optional[torch.Tensor], w_out: torch.Tensor,
                      norms: Optional[torch.Tensor], epsilon: float = 1e-6) -> None:
    _check(lib().bsmm_l2_normalize(h, _dev_ptr(w, "w"), _dev_ptr(gain, "gain"), _dev_ptr(w_out, "w_out"),
                                   _dev_ptr(norms, "norms"), float(epsilon), DTYPE_CODE[w.dtype],
                                   DTYPE_CODE[w_out.dtype], _stream(w)), "bsmm_l2_normalize")


def bsmm_l2_normalize_grad(h, dy: torch.Tensor, w: torch.Tensor, gain: Optional[torch.Tensor], dw: torch.Tensor,
                           dgain: Optional[torch.Tensor], epsilon: float = 1e-6) -> None:
    _check(lib().bsmm_l2_normalize_grad(h, _dev_ptr(dy, "dy"), _dev_ptr(w, "w"), _dev_ptr(gain, "gain"),
                                        _dev_ptr(dw, "dw"), _dev_ptr(dgain, "dgain"), float(epsilon),
                                        DTYPE_CODE[dy.dtype], DTYPE_CODE[w.dtype], _stream(w)),
           "bsmm_l2_normalize_grad")


class _L2NormalizeFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, bsmm, w, gain, epsilon, dtype):
        out = torch.empty(w.shape, dtype=dtype, device=w.device)
        bsmm_l2_normalize(bsmm.handle, w, gain, out, None, epsilon)
        ctx.save_for_backward(w, gain if gain is not None else torch.empty(0))
        ctx.bsmm, ctx.eps, ctx.has_gain = bsmm, epsilon, gain is not None
        return out

    @staticmethod
    def backward(ctx, dy):
        w, gain = ctx.saved_tensors
        gain = gain if ctx.has_gain else None
        dw = torch.empty(w.shape, dtype=torch.float32, device=w.device)
        dgain = torch.empty_like(gain) if gain is not None else None
        bsmm_l2_normalize_grad(ctx.bsmm.handle, dy.contiguous(), w, gain, dw, dgain, ctx.eps)
        return None, dw.to(w.dtype), dgain, None, None


# ---- BlocksparseMatMul --------------------------------------------------------------
class _Handle:
    def __init__(self, h):
        self.h = h

    def __del__(self):
        try:
            if self.h:
                lib().bsmm_destroy(self.h)
        except Exception:
            pass


class _BsmmFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, bsmm, x, w, dw_dtype):
        ctx.bsmm = bsmm
        ctx.dw_dtype = dw_dtype
        ctx.save_for_backward(x, w)
        return bsmm.fprop(x, w)

    @staticmethod
    def backward(ctx, dy):
        x, w = ctx.saved_tensors
        bsmm = ctx.bsmm
        dy = dy.contiguous()
        dx = bsmm.bprop(dy, w) if ctx.needs_input_grad[1] else None
        dw = bsmm.updat([x], [dy], dw_dtype=ctx.dw_dtype).to(w.dtype) if ctx.needs_input_grad[2] else None
        return None, dx, dw, None


class BlocksparseMatMul:
    """y = x . W for a block-sparse W (see include/bsmm.h for the exact conventions).

    layout        2-D array of zeros and ones, shape (C/b, K/b); row = input block c.
    block_size    8, 16 or 32.
    feature_axis  1: activations (N, features); 0: (features, N).
    """

    def __init__(self, layout, block_size: int = 32, feature_axis: int = 1):
        self.layout = np.ascontiguousarray(np.asarray(layout), dtype=np.uint8)
        self.block_size = int(block_size)
        self.feature_axis = int(feature_axis)
        self._h = _Handle(bsmm_create(self.layout, self.block_size, self.feature_axis))
        info = bsmm_plan_info(self._h.h)
        self.R, self.S, self.nnz = info["R"], info["S"], info["nnz"]
        self.C = self.R * self.block_size
        self.K = self.S * self.block_size

    @property
    def handle(self):
        return self._h.h

    # shape helpers (N = minibatch)
    @property
    def w_shape(self):
        return bsmm_w_shape(self.handle)

    def i_shape(self, N: int):
        return bsmm_i_shape(self.handle, N)

    def o_shape(self, N: int):
        return bsmm_o_shape(self.handle, N)

    def block_coord(self, block: int):
        return bsmm_block_coord(self.handle, block)

    def kernel_name(self, pass_: str, N: int, dtype: torch.dtype = torch.float32, group: int = 1) -> str:
        """Kernel family `pass_` ("fprop", "bprop", "updat", "identity") launches at N."""
        return bsmm_kernel_name(self.handle, PASS[pass_], N, dtype, group)

    def force_kernel(self, pass_: str, name: Optional[str]) -> None:
        """Testing and tuning: launch the named kernel family for `pass_` (None: automatic)."""
        bsmm_force_kernel(self.handle, PASS[pass_], name)

    def _N(self, t: torch.Tensor, feats: int, what: str) -> int:
        if t.dim() != 2:
            raise ValueError(f"{what} must be 2-D")
        if self.feature_axis == 1:
            if t.shape[1] != feats:
                raise ValueError(f"{what} has {t.shape[1]} features, expected {feats}")
            return t.shape[0]
        if t.shape[0] != feats:
            raise ValueError(f"{what} has {t.shape[0]} features, expected {feats}")
        return t.shape[1]

    def _check_w(self, w: torch.Tensor, dtype):
        if tuple(w.shape) != tuple(self.w_shape):
            raise ValueError(f"w has shape {tuple(w.shape)}, expected {self.w_shape}")
        if w.dtype != dtype:
            raise ValueError("w and the activations must share a dtype")

    def identity_init(self, gpu: bool = False, dtype=torch.float32, device=None):
        """Identity on present diagonal blocks, zero elsewhere.  gpu=True runs the device
        kernel and returns a device tensor; gpu=False returns the initial value as a host
        numpy array built from the layout's block coordinates."""
        if gpu:
            device = device or torch.device("cuda", torch.cuda.current_device())
            w = torch.empty(self.w_shape, dtype=dtype, device=device)
            bsmm_identity_init(self.handle, w)
            return w
        b = self.block_size
        w = np.zeros(self.w_shape, dtype=np.float32)
        eye = np.eye(b, dtype=np.float32)
        for t in range(self.nnz):
            c, k = self.block_coord(t)
            if c == k:
                w[t] = eye
        return w

    def fprop(self, x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
        N = self._N(x, self.C, "x")
        self._check_w(w, x.dtype)
        y = torch.empty(self.o_shape(N), dtype=x.dtype, device=x.device)
        bsmm_fprop(self.handle, x, w, y, N)
        return y

    def bprop(self, dy: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
        N = self._N(dy, self.K, "dy")
        self._check_w(w, dy.dtype)
        dx = torch.empty(self.i_shape(N), dtype=dy.dtype, device=dy.device)
        bsmm_bprop(self.handle, dy, w, dx, N)
        return dx

    def updat(self, xs: Sequence[torch.Tensor], dys: Sequence[torch.Tensor], dw_dtype=torch.float32,
              out: Optional[torch.Tensor] = None, accumulate: bool = False) -> torch.Tensor:
        """dW summed over the given steps (1 to 8), written in dw_dtype.  accumulate=True
        adds that sum to `out` (required) instead of overwriting it, so sequences of more
        than 8 steps sharing one weight sum their groups into one gradient."""
        if accumulate and out is None:
            raise ValueError("accumulate needs the gradient to add into (out=)")
        if not 1 <= len(xs) <= 8 or len(xs) != len(dys):
            raise ValueError("updat takes 1 to 8 (x, dy) pairs")
        N = self._N(xs[0], self.C, "x")
        for x, dy in zip(xs, dys):
            if self._N(x, self.C, "x") != N or self._N(dy, self.K, "dy") != N:
                raise ValueError("every step must have the same minibatch")
            if x.dtype != xs[0].dtype or dy.dtype != xs[0].dtype:
                raise ValueError("all steps must share a dtype")
        if out is not None:
            if tuple(out.shape) != tuple(self.w_shape):
                raise ValueError(f"out has shape {tuple(out.shape)}, expected {self.w_shape}")
            _need(out, "out", self.w_shape, None, xs[0].device)
        dw = out if out is not None else torch.empty(self.w_shape, dtype=dw_dtype, device=xs[0].device)
        bsmm_updat(self.handle, xs, dys, dw, N, accumulate=accumulate)
        return dw

    def l2_normalize(self, w: torch.Tensor, gain: Optional[torch.Tensor] = None, epsilon: float = 1e-6,
                     dtype=torch.float32) -> torch.Tensor:
        """Weight normalisation of the stored blocks per output feature (README,
        BlocksparseMatMul.l2_normalize): w * gain[o] / sqrt(max(sum over the output
        feature's column of w^2, epsilon)); gain: float32 (K,) or None; the result in
        `dtype`.  Differentiable in w and gain."""
        self._check_w(w, w.dtype)
        if gain is not None and (gain.dtype != torch.float32 or tuple(gain.shape) != (self.K,)):
            raise ValueError("gain must be a float32 vector of the K output features")
        return _L2NormalizeFunction.apply(self, w, gain, epsilon, dtype)

    def __call__(self, x: torch.Tensor, w: torch.Tensor, dw_dtype=torch.float32) -> torch.Tensor:
        """y = x . W, differentiable in x and w (bprop and updat kernels)."""
        return _BsmmFunction.apply(self, x, w, dw_dtype)


def group_param_grads(bsmm: BlocksparseMatMul, xs: Sequence[torch.Tensor], dys: Sequence[torch.Tensor],
                      dw_dtype=torch.float32, group_size: int = 8) -> torch.Tensor:
    """One weight gradient for the steps that share W: the sum of the per-step dWs.  The
    steps are taken group_size (1 to 8, the README's group_param_grads limit) at a time,
    one grouped updat launch each (fp32 accumulation within a launch); the first launch
    writes the gradient and every later one adds its group's sum into it."""
    if not 1 <= group_size <= 8:
        raise ValueError("group_size must be in [1, 8]")
    if len(xs) == 0 or len(xs) != len(dys):
        raise ValueError("xs and dys must be non-empty and of equal length")
    dw = bsmm.updat(xs[:group_size], dys[:group_size], dw_dtype=dw_dtype)
    for t in range(group_size, len(xs), group_size):
        bsmm.updat(xs[t:t + group_size], dys[t:t + group_size], out=dw, accumulate=True)
    return dw


# ---- SparseProj (README, "API Documentation" › blocksparse.matmul › SparseProj) ---------
def _proj_call(fn: str, h, *tensors_and_n, fa: int):
    *ts, N = tensors_and_n
    dt = ts[0].dtype
    for t in ts:
        if t.dtype != dt:
            raise ValueError("SparseProj operands must share a dtype")
    ptrs = [_dev_ptr(t, f"arg{i}") for i, t in enumerate(ts)]
    _check(getattr(lib(), fn)(h, *ptrs, N, fa, DTYPE_CODE[dt], _stream(ts[0])), fn)


def bsmm_proj_gather(h, x: torch.Tensor, y: torch.Tensor, N: int, fa: int = 1) -> None:
    _proj_call("bsmm_proj_gather", h, x, y, N, fa=fa)


def bsmm_proj_scatter(h, x: torch.Tensor, y: torch.Tensor, N: int, fa: int = 1) -> None:
    _proj_call("bsmm_proj_scatter", h, x, y, N, fa=fa)


def bsmm_proj_scatter_add(h, x: torch.Tensor, y: torch.Tensor, z: torch.Tensor, N: int, fa: int = 1) -> None:
    _proj_call("bsmm_proj_scatter_add", h, x, y, z, N, fa=fa)


def bsmm_proj_scatter_mul(h, x: torch.Tensor, y: torch.Tensor, z: torch.Tensor, N: int, fa: int = 1) -> None:
    _proj_call("bsmm_proj_scatter_mul", h, x, y, z, N, fa=fa)


def bsmm_proj_gather_mul(h, a: torch.Tensor, b: torch.Tensor, g: torch.Tensor, N: int, fa: int = 1) -> None:
    _proj_call("bsmm_proj_gather_mul", h, a, b, g, N, fa=fa)


class _ProjGather(torch.autograd.Function):
    @staticmethod
    def forward(ctx, proj, x):
        ctx.proj = proj
        return proj._gather(x)

    @staticmethod
    def backward(ctx, dy):
        return None, ctx.proj._scatter(dy.contiguous())


class _ProjScatter(torch.autograd.Function):
    @staticmethod
    def forward(ctx, proj, x):
        ctx.proj = proj
        return proj._scatter(x)

    @staticmethod
    def backward(ctx, dy):
        return None, ctx.proj._gather(dy.contiguous())


class _ProjScatterAdd(torch.autograd.Function):
    @staticmethod
    def forward(ctx, proj, x, y):
        ctx.proj = proj
        return proj._scatter_add(x, y)

    @staticmethod
    def backward(ctx, dz):
        dz = dz.contiguous()
        return None, dz, ctx.proj._gather(dz)


class _ProjScatterMul(torch.autograd.Function):
    @staticmethod
    def forward(ctx, proj, x, y):
        ctx.proj = proj
        ctx.save_for_backward(x, y)
        return proj._scatter_mul(x, y)

    @staticmethod
    def backward(ctx, dz):
        x, y = ctx.saved_tensors
        dz = dz.contiguous()
        return None, ctx.proj._scatter_mul(dz, y), ctx.proj._gather_mul(dz, x)


class SparseProj:
    """Dense <-> projected feature maps (README, SparseProj(nhidden, nproj=None,
    proj_stride=None, block_size=32, gather_lut=None)) over a one-to-one map lut of nproj
    dense features: gather(x) = x[:, lut], scatter(x) puts the projected features back
    (zeros elsewhere), scatter_add(x, y) / scatter_mul(x, y) add / multiply y into x at
    lut.  Without gather_lut the map is nproj // block_size blocks of block_size
    consecutive features, block j at j * proj_stride (nproj defaults to nhidden,
    proj_stride to block_size).  feature_axis (an addition of this binding): 1 for (N,
    features) activations, 0 for (features, N).  Every op is differentiable; the backward
    ops are the same kernels (the map is one-to-one: no atomics)."""

    def __init__(self, nhidden: int, nproj: Optional[int] = None, proj_stride: Optional[int] = None,
                 block_size: int = 32, gather_lut=None, feature_axis: int = 1):
        h = ctypes.c_void_p()
        if gather_lut is not None:
            lut = np.ascontiguousarray(np.asarray(gather_lut), dtype=np.int32)
            if lut.ndim != 1 or (nproj is not None and nproj != lut.size):
                raise ValueError("gather_lut must be 1-D with nproj entries")
            _check(lib().bsmm_proj_create(ctypes.byref(h), int(nhidden), int(lut.size), 0, 0,
                                          lut.ctypes.data_as(ctypes.c_void_p)), "bsmm_proj_create")
        else:
            _check(lib().bsmm_proj_create(ctypes.byref(h), int(nhidden), int(nproj or 0), int(proj_stride or 0),
                                          int(block_size), None), "bsmm_proj_create")
        self.handle = h
        if feature_axis not in (0, 1):
            raise ValueError("feature_axis must be 0 or 1")
        self.feature_axis = feature_axis
        nh, npj = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().bsmm_proj_info(h, ctypes.byref(nh), ctypes.byref(npj)), "bsmm_proj_info")
        self.nhidden, self.nproj = nh.value, npj.value

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.bsmm_proj_destroy(h)
            self.handle = None

    @property
    def gather_lut(self) -> np.ndarray:
        out = np.empty(self.nproj, dtype=np.int32)
        _check(lib().bsmm_proj_lut(self.handle, out.ctypes.data_as(ctypes.c_void_p), self.nproj), "bsmm_proj_lut")
        return out

    def _shape(self, N: int, feats: int):
        return (N, feats) if self.feature_axis == 1 else (feats, N)

    def _N(self, t: torch.Tensor, feats: int, what: str) -> int:
        if t.dim() != 2:
            raise ValueError(f"{what} must be 2-D")
        fdim, ndim = (1, 0) if self.feature_axis == 1 else (0, 1)
        if t.shape[fdim] != feats:
            raise ValueError(f"{what} has {t.shape[fdim]} features, expected {feats}")
        return t.shape[ndim]

    def _gather(self, x):
        N = self._N(x, self.nhidden, "x")
        y = torch.empty(self._shape(N, self.nproj), dtype=x.dtype, device=x.device)
        bsmm_proj_gather(self.handle, x, y, N, self.feature_axis)
        return y

    def _scatter(self, x):
        N = self._N(x, self.nproj, "x")
        y = torch.empty(self._shape(N, self.nhidden), dtype=x.dtype, device=x.device)
        bsmm_proj_scatter(self.handle, x, y, N, self.feature_axis)
        return y

    def _scatter_add(self, x, y):
        N = self._N(x, self.nhidden, "x")
        if self._N(y, self.nproj, "y") != N:
            raise ValueError("x and y differ in minibatch")
        z = torch.empty_like(x)
        bsmm_proj_scatter_add(self.handle, x, y, z, N, self.feature_axis)
        return z

    def _scatter_mul(self, x, y):
        N = self._N(x, self.nhidden, "x")
        if self._N(y, self.nproj, "y") != N:
            raise ValueError("x and y differ in minibatch")
        z = torch.empty_like(x)
        bsmm_proj_scatter_mul(self.handle, x, y, z, N, self.feature_axis)
        return z

    def _gather_mul(self, a, b):
        N = self._N(a, self.nhidden, "a")
        if self._N(b, self.nhidden, "b") != N:
            raise ValueError("a and b differ in minibatch")
        g = torch.empty(self._shape(N, self.nproj), dtype=a.dtype, device=a.device)
        bsmm_proj_gather_mul(self.handle, a, b, g, N, self.feature_axis)
        return g

    def gather(self, x: torch.Tensor) -> torch.Tensor:
        return _ProjGather.apply(self, x.contiguous())

    def scatter(self, x: torch.Tensor) -> torch.Tensor:
        return _ProjScatter.apply(self, x.contiguous())

    def scatter_add(self, x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
        return _ProjScatterAdd.apply(self, x.contiguous(), y.contiguous())

    def scatter_mul(self, x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
        return _ProjScatterMul.apply(self, x.contiguous(), y.contiguous())


# ---- BlocksparseConv (README, "API Documentation" › blocksparse.conv) -----------------------
def bsmm_conv_fprop(h, F: torch.Tensor, I: torch.Tensor, O: torch.Tensor, N: int) -> None:
    if F.dtype != I.dtype or O.dtype != I.dtype:
        raise ValueError("F, I and O must share a dtype")
    _check(lib().bsmm_conv_fprop(h, _dev_ptr(F, "F"), _dev_ptr(I, "I"), _dev_ptr(O, "O"), N, DTYPE_CODE[I.dtype],
                                 _stream(I)), "bsmm_conv_fprop")


def bsmm_conv_bprop(h, F: torch.Tensor, dO: torch.Tensor, dI: torch.Tensor, N: int) -> None:
    if F.dtype != dO.dtype or dI.dtype != dO.dtype:
        raise ValueError("F, dO and dI must share a dtype")
    _check(lib().bsmm_conv_bprop(h, _dev_ptr(F, "F"), _dev_ptr(dO, "dO"), _dev_ptr(dI, "dI"), N,
                                 DTYPE_CODE[dO.dtype], _stream(dO)), "bsmm_conv_bprop")


def bsmm_conv_updat(h, I: torch.Tensor, dO: torch.Tensor, dF: torch.Tensor, N: int) -> None:
    """dF = the filter gradient; allocates the contraction-split workspace the library asks for."""
    if I.dtype != dO.dtype or dF.dtype != torch.float32:
        raise ValueError("I and dO must share a dtype; dF is float32")
    nb = ctypes.c_size_t()
    _check(lib().bsmm_conv_workspace_size(h, N, DTYPE_CODE[I.dtype], ctypes.byref(nb)), "bsmm_conv_workspace_size")
    ws = torch.empty(nb.value, dtype=torch.uint8, device=I.device) if nb.value else None
    _check(lib().bsmm_conv_updat(h, _dev_ptr(I, "I"), _dev_ptr(dO, "dO"), _dev_ptr(dF, "dF"), N,
                                 DTYPE_CODE[I.dtype], _dev_ptr(ws, "ws"), nb.value, _stream(I)), "bsmm_conv_updat")


class _ConvFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, conv, F, I):
        ctx.conv = conv
        ctx.save_for_backward(F, I)
        return conv.fprop(F, I)

    @staticmethod
    def backward(ctx, dO):
        F, I = ctx.saved_tensors
        conv = ctx.conv
        dO = dO.contiguous()
        dF = conv.updat(I, dO).to(F.dtype) if ctx.needs_input_grad[1] else None
        dI = conv.bprop(F, dO) if ctx.needs_input_grad[2] else None
        return None, dF, dI


class BlocksparseConv:
    """Convolution with a filter only for blocks of channels (README, BlocksparseConv(BCK,
    TRS, DHW, MPQ=None, strides=(1,1,1), dilates=(1,1,1), padding="SAME",
    edge_bias=False)).  BCK: one ((c0, c1, ...), (k0, k1, ...)) pair per block (every
    block the same sizes Bc, Bk <= 64); TRS / DHW / strides / dilates: 1 to 3 spatial
    dims; padding "SAME", "VALID", an int or a tuple of ints.  Activations (N, C, *DHW)
    and (N, K, *MPQ) with C, K one past the largest channel index; the filter
    (nblocks, Bc, *TRS, Bk).  edge_bias and MPQ (transposed convolution) are not
    provided."""

    def __init__(self, BCK, TRS, DHW, MPQ=None, strides=(1, 1, 1), dilates=(1, 1, 1), padding="SAME",
                 edge_bias=False):
        if edge_bias:
            raise NotImplementedError("edge_bias is not provided")
        nd = len(tuple(DHW))
        if len(tuple(TRS)) != nd:
            raise ValueError("TRS and DHW must have the same number of dims")
        cl = np.ascontiguousarray([blk[0] for blk in BCK], dtype=np.int32)
        kl = np.ascontiguousarray([blk[1] for blk in BCK], dtype=np.int32)
        if cl.ndim != 2 or kl.ndim != 2:
            raise ValueError("every block must list the same numbers of input and output channels")
        self.nblocks, self.Bc = cl.shape
        self.Bk = kl.shape[1]
        self.C = int(cl.max()) + 1
        self.K = int(kl.max()) + 1
        self.nd = nd

        def pad3(v, fill):
            v = tuple(int(a) for a in (v if isinstance(v, (tuple, list)) else (v,) * nd))
            v = v[-nd:] if len(v) >= nd else v
            return (fill,) * (3 - len(v)) + v

        arr = lambda v: (ctypes.c_int64 * 3)(*v)
        if isinstance(padding, str):
            mode, pads = {"SAME": 0, "VALID": 1}[padding.upper()], (0, 0, 0)
        else:
            mode, pads = 2, pad3(padding, 0)
        h = ctypes.c_void_p()
        _check(lib().bsmm_conv_create(ctypes.byref(h), self.nblocks, self.Bc, self.Bk,
                                      cl.ctypes.data_as(ctypes.c_void_p), kl.ctypes.data_as(ctypes.c_void_p),
                                      self.C, self.K, arr(pad3(TRS, 1)), arr(pad3(DHW, 1)), arr(pad3(strides, 1)),
                                      arr(pad3(dilates, 1)), mode, arr(pads)), "bsmm_conv_create")
        self.handle = h
        m3, p3 = (ctypes.c_int64 * 3)(), (ctypes.c_int64 * 3)()
        _check(lib().bsmm_conv_geometry(h, m3, p3), "bsmm_conv_geometry")
        self.TRS, self.DHW = tuple(TRS), tuple(DHW)
        self.MPQ = tuple(m3[3 - nd:])
        self.pads = tuple(p3[3 - nd:])
        if MPQ is not None and tuple(MPQ) != self.MPQ:
            raise ValueError(f"MPQ {tuple(MPQ)} differs from the output size {self.MPQ} (transposed convolution "
                             "is not provided)")

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.bsmm_conv_destroy(h)
            self.handle = None

    def kernel_name(self, pass_: str, dtype=torch.bfloat16) -> str:
        """Kernel family a pass ("fprop", "bprop", "updat") launches: "matrix_core",
        "matrix_core_gather" or "direct"."""
        name = ctypes.c_char_p()
        _check(lib().bsmm_conv_kernel_name(self.handle, {"fprop": 0, "bprop": 1, "updat": 2}[pass_],
                                           DTYPE_CODE[dtype], ctypes.byref(name)), "bsmm_conv_kernel_name")
        return name.value.decode()

    def f_shape(self, block=None):
        one = (self.Bc,) + self.TRS + (self.Bk,)
        return one if block is not None else (self.nblocks,) + one

    def i_shape(self, N):
        return (N, self.C) + self.DHW

    def o_shape(self, N):
        return (N, self.K) + self.MPQ

    def _check_act(self, t, shape, what):
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")

    def fprop(self, F, I):
        N = I.shape[0]
        self._check_act(I, self.i_shape(N), "I")
        self._check_act(F, self.f_shape(), "F")
        O = torch.empty(self.o_shape(N), dtype=I.dtype, device=I.device)
        bsmm_conv_fprop(self.handle, F.contiguous(), I.contiguous(), O, N)
        return O

    def bprop(self, F, dO):
        N = dO.shape[0]
        self._check_act(dO, self.o_shape(N), "dO")
        dI = torch.empty(self.i_shape(N), dtype=dO.dtype, device=dO.device)
        bsmm_conv_bprop(self.handle, F.contiguous(), dO.contiguous(), dI, N)
        return dI

    def updat(self, I, dO):
        N = I.shape[0]
        self._check_act(I, self.i_shape(N), "I")
        self._check_act(dO, self.o_shape(N), "dO")
        dF = torch.empty(self.f_shape(), dtype=torch.float32, device=I.device)
        bsmm_conv_updat(self.handle, I.contiguous(), dO.contiguous(), dF, N)
        return dF

    def __call__(self, F, I):
        return _ConvFn.apply(self, F, I)
