"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds every source of libbsmm with the sanitizers on the host code only (the device
code is compiled as usual, without them), links it with tests/sanitize/host_driver.cpp, and runs
the driver: the layout compiler over many layouts (every block size and feature axis,
empty to full, long lists, a band) with the tables' invariants checked, and every C-ABI
argument check with fake device pointers.  No GPU is needed or used.  The test fails on
a failed check or on any sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_matrix_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]


def _build():
    import concurrent.futures
    from block_sparse_matrix_amd import build as B
    os.makedirs(OUT, exist_ok=True)
    common = ["-O1", "-g", "-std=c++17", "-fPIC", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]

    def one(src):
        obj = os.path.join(OUT, src + ".o")
        lang = ["-x", "hip", *B.DEVICE] if src.endswith(".hip") else ["-x", "c++"]
        cmd = [HIPCC, *common, *SAN, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(one, B.SOURCES))
    drv = os.path.join(OUT, "host_driver")
    cmd = [HIPCC, f"--offload-arch={B.ARCH}", *common, *SAN, "-x", "c++",
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), "-x", "none", *objs, "-o", drv]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return drv


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_code_under_sanitizers():
    drv = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([drv], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "ERROR: LeakSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0 and "host driver: ok" in out, out[-4000:]
