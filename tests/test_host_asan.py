"""The library's host code under AddressSanitizer: the codebook enumeration, the pack
builder, argument validation and the workspace plans.

build.py's asan variant (libglq_mi355x_asan.so) compiles the host code of every source
with AddressSanitizer (device code is not instrumented).  The CPU tests of the ABI and
of the pack builder run again against it in a subprocess, with the clang ASan runtime
loaded first (prepended to any LD_PRELOAD already set) and leak checks off (the
interpreter's own allocations are not this library's).  Any ASan report aborts the
subprocess and fails this test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "e8_lattice_codebook_amd", "libglq_mi355x_asan.so")


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_host_code_under_asan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime in this image")
    if not os.path.exists(LIB):
        pytest.skip("libglq_mi355x_asan.so is not built (e8_lattice_codebook_amd/build.py --variant asan)")
    with open(LIB, "rb") as fh:
        assert b"__asan_" in fh.read(), "the asan variant carries no ASan instrumentation"
    pre = os.environ.get("LD_PRELOAD", "")
    env = dict(os.environ, GLQ_LIB_VARIANT="asan", ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               LD_PRELOAD=rt + (":" + pre if pre else ""))
    probe = "import e8_lattice_codebook_amd._lib as l; l.load(); print(l.LIB_PATH)"
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.strip().endswith("libglq_mi355x_asan.so"), r.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "tests/test_pack.py", "-m", "not gpu",
                        "-q", "-x", "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
