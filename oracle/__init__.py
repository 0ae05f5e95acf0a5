"""CPU oracle for the block-sparse matmul -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg import this
package.  The product (block_sparse_matrix_amd and libbsmm.so) never does, and the
two share no code.

The arithmetic lives in bsmm_oracle.c (plain C, fp64, OpenMP over output blocks);
this module compiles it with gcc and marshals numpy arrays in and out.  Each
function states the passage of the kiteco/blocksparse README it follows.

Inputs are raw storage: float32 arrays for fp32, uint16 bit patterns for bfloat16
and float16 (see synth.to_bits).  Outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bsmm_oracle.c")
LIB = os.path.join(HERE, "libbsmm_oracle.so")

DT = {"f32": 0, "bf16": 1, "f16": 2}

_lib = None


def build(src: str = SRC, out: str = LIB, extra_flags: Sequence[str] = ()) -> str:
    """Compile the oracle with gcc (-O2 -fopenmp).  Returns the library path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", *extra_flags,
           "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: Optional[str] = None):
    """Load (building first if absent) the oracle library and declare its signatures."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or LIB
    if not os.path.exists(p) or (path is None and os.path.getmtime(p) < os.path.getmtime(SRC)):
        build(out=p)
    lib = ctypes.CDLL(p)
    i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    u8p = ctypes.c_void_p
    lib.orc_decode.restype = ctypes.c_double
    lib.orc_decode.argtypes = [vp, i64, ctypes.c_int]
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_nnz.restype = i64
    lib.orc_nnz.argtypes = [u8p, i64, i64]
    for name in ("orc_fprop", "orc_bprop"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [u8p, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, i64, dp]
    lib.orc_updat.restype = ctypes.c_int
    lib.orc_updat.argtypes = [u8p, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                              vp, vp, ctypes.c_int, i64, vp, i64, dp]
    lib.orc_identity.restype = ctypes.c_int
    lib.orc_identity.argtypes = [u8p, i64, i64, ctypes.c_int, dp]
    lib.orc_block_coord.restype = ctypes.c_int
    lib.orc_block_coord.argtypes = [u8p, i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    if path is None:
        _lib = lib
    return lib


def _dt_of(a: np.ndarray, dtype: Optional[str]) -> int:
    if dtype is not None:
        return DT[dtype]
    if a.dtype == np.float32:
        return DT["f32"]
    raise ValueError("16-bit inputs need an explicit dtype ('bf16' or 'f16')")


def _check_storage(a: np.ndarray, dt: int):
    want = np.float32 if dt == 0 else np.uint16
    if a.dtype != want:
        raise TypeError(f"expected {want} storage, got {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError("arrays must be C-contiguous")


def _layout(layout) -> np.ndarray:
    L = np.ascontiguousarray(layout, dtype=np.uint8)
    if L.ndim != 2:
        raise ValueError("layout must be 2-D")
    return L


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def nnz(layout) -> int:
    L = _layout(layout)
    return int(load().orc_nnz(_ptr(L), L.shape[0], L.shape[1]))


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact decode of stored values to float64 (one C call per element; small arrays only)."""
    lib = load()
    a = np.ascontiguousarray(bits)
    out = np.empty(a.size, dtype=np.float64)
    flat = a.reshape(-1)
    for t in range(flat.size):
        out[t] = lib.orc_decode(_ptr(flat), t, DT[dtype])
    return out.reshape(a.shape)


def fprop(layout, block: int, fa: int, x: np.ndarray, w: np.ndarray, N: int,
          dtype: Optional[str] = None, lib=None) -> np.ndarray:
    """y = x . W over the present blocks (README, blocksparse.matmul, BlocksparseMatMul.__call__)."""
    lib = lib or load()
    L = _layout(layout)
    R, S = L.shape
    dt = _dt_of(x, dtype)
    _check_storage(x, dt), _check_storage(w, dt)
    K = S * block
    y = np.empty((N, K) if fa == 1 else (K, N), dtype=np.float64)
    rc = lib.orc_fprop(_ptr(L), R, S, block, fa, dt, _ptr(x), _ptr(w), N, _ptr(y))
    if rc != 0:
        raise ValueError(f"orc_fprop failed ({rc})")
    return y


def bprop(layout, block: int, fa: int, dy: np.ndarray, w: np.ndarray, N: int,
          dtype: Optional[str] = None, lib=None) -> np.ndarray:
    """dx = dy . W^T over the present blocks (the input gradient of __call__)."""
    lib = lib or load()
    L = _layout(layout)
    R, S = L.shape
    dt = _dt_of(dy, dtype)
    _check_storage(dy, dt), _check_storage(w, dt)
    C = R * block
    dx = np.empty((N, C) if fa == 1 else (C, N), dtype=np.float64)
    rc = lib.orc_bprop(_ptr(L), R, S, block, fa, dt, _ptr(dy), _ptr(w), N, _ptr(dx))
    if rc != 0:
        raise ValueError(f"orc_bprop failed ({rc})")
    return dx


def updat(layout, block: int, fa: int, xs: Sequence[np.ndarray], dys: Sequence[np.ndarray], N: int,
          dtype: Optional[str] = None, ids: Optional[Sequence[int]] = None, lib=None) -> np.ndarray:
    """dW[id(c,k)] = sum_t x_t[:, c-block]^T . dy_t[:, k-block] (weight gradient, grouped over t)."""
    lib = lib or load()
    L = _layout(layout)
    R, S = L.shape
    if len(xs) != len(dys) or len(xs) < 1:
        raise ValueError("xs and dys must be non-empty and of equal length")
    dt = _dt_of(xs[0], dtype)
    for a in list(xs) + list(dys):
        _check_storage(a, dt)
    G = len(xs)
    xp = (ctypes.c_void_p * G)(*[a.ctypes.data for a in xs])
    dp = (ctypes.c_void_p * G)(*[a.ctypes.data for a in dys])
    if ids is None:
        n_out = int(lib.orc_nnz(_ptr(L), R, S))
        idp, nids = None, 0
    else:
        ida = np.ascontiguousarray(ids, dtype=np.int64)
        n_out = ida.size
        idp, nids = _ptr(ida), ida.size
    dw = np.empty((n_out, block, block), dtype=np.float64)
    rc = lib.orc_updat(_ptr(L), R, S, block, fa, dt, xp, dp, G, N, idp, nids, _ptr(dw))
    if rc != 0:
        raise ValueError(f"orc_updat failed ({rc})")
    return dw


def updat_accumulate(layout, block: int, fa: int, dw0: np.ndarray, dw_dtype: str, xs: Sequence[np.ndarray],
                     dys: Sequence[np.ndarray], N: int, dtype: Optional[str] = None, lib=None) -> np.ndarray:
    """dW0 + sum_t x_t[:, c-block]^T . dy_t[:, k-block]: the weight gradient added into a
    stored one.  Steps that share one weight contribute one summed gradient (README,
    group_param_grads, which combines up to 8 of them per product); a sequence longer
    than one group adds its groups' sums into the same gradient.  dw0 is raw storage of
    dw_dtype ("f32": float32 values, "bf16" / "f16": uint16 bit patterns), decoded
    exactly by the oracle's decoder."""
    lib = lib or load()
    base = np.asarray(dw0, dtype=np.float64) if dw_dtype == "f32" else decode(dw0, dw_dtype)
    return base + updat(layout, block, fa, xs, dys, N, dtype, lib=lib)


def identity(layout, block: int, lib=None) -> np.ndarray:
    """identity_init: I_b on present diagonal blocks, zero elsewhere (README, identity_init)."""
    lib = lib or load()
    L = _layout(layout)
    R, S = L.shape
    n = int(lib.orc_nnz(_ptr(L), R, S))
    w = np.empty((n, block, block), dtype=np.float64)
    if lib.orc_identity(_ptr(L), R, S, block, _ptr(w)) != 0:
        raise ValueError("orc_identity failed")
    return w


def block_coord(layout, block_id: int, lib=None):
    """(c, k) of a block id under the row-major numbering of the layout's nonzeros."""
    lib = lib or load()
    L = _layout(layout)
    c, k = ctypes.c_int64(), ctypes.c_int64()
    if lib.orc_block_coord(_ptr(L), L.shape[0], L.shape[1], block_id, ctypes.byref(c), ctypes.byref(k)) != 0:
        raise IndexError(block_id)
    return int(c.value), int(k.value)


def num_threads(lib=None) -> int:
    return int((lib or load()).orc_num_threads())
