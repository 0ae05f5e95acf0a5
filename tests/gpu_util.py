"""Shared helpers for the GPU parity tests: tolerances and comparison."""
import numpy as np
import torch

# Max relative error, infinity-norm: max|gpu - oracle| / max|oracle|.
#   fp32 storage, fp32 accumulate:                 1e-5
#   bf16 / f16 storage, fp32 accumulate, rounded:  2e-2
TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 2e-2}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def rel_err(got: torch.Tensor, ref: np.ndarray) -> float:
    g = got.detach().float().cpu().double().numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), "non-finite values in GPU output"
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    d = float(np.max(np.abs(g - ref))) if ref.size else 0.0
    if m == 0.0:
        return d
    return d / m


def assert_close(got, ref, dtype, what=""):
    e = rel_err(got, ref)
    assert e <= TOL[dtype], f"{what}: max rel err {e:.3e} > {TOL[dtype]:.0e}"
    return e


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda").contiguous()
