"""The oracle against its pins (CPU only).  See pins.py for what each pin checks."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", [p for p in pins.ALL_PINS if p is not pins.pin_dense_masked],
                         ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fa", [0, 1])
@pytest.mark.parametrize("b", [8, 16, 32])
def test_dense_masked(lib, b, fa, dtype):
    pins.pin_dense_masked(lib, b=b, fa=fa, dtype=dtype, R=3, S=5, N=7, seed=b + fa)


def test_dense_masked_tall_and_empty(lib):
    # C != K in both directions, and an all-zero layout (nnz = 0).
    pins.pin_dense_masked(lib, b=8, fa=1, R=6, S=2, N=3, seed=11)
    pins.pin_dense_masked(lib, b=8, fa=0, R=1, S=7, N=3, seed=12)
    import numpy as np
    L = np.zeros((2, 3), dtype=np.uint8)
    x = np.ones((4, 16), dtype=np.float32)
    w = np.zeros((0, 8, 8), dtype=np.float32)
    assert (oracle.fprop(L, 8, 1, x, w, 4) == 0).all()
    assert oracle.nnz(L) == 0


def test_thread_count_does_not_change_results(lib, monkeypatch):
    # sums are never split across threads; compare with a single-threaded build run
    import subprocess, sys, os, json
    code = ("import sys; sys.path.insert(0, %r); import numpy as np, oracle, synth;"
            "rng=np.random.default_rng(3); L=(rng.random((4,4))<0.5).astype(np.uint8);"
            "P=synth.random_problem(rng,L,16,9,1,'f32');"
            "y=oracle.fprop(L,16,1,synth.to_bits(P.xs[0]),synth.to_bits(P.w),9);"
            "print(float(np.sum(y*np.arange(y.size).reshape(y.shape))).hex())") % os.path.dirname(os.path.dirname(__file__))
    outs = set()
    for t in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=t)
        outs.add(subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                                check=True).stdout.strip())
    assert len(outs) == 1
