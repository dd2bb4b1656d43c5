"""Build the gfx950 HIP library libglq_mi355x.so in-tree with hipcc.

Every call compiles every source again (object files go to _build/ at the repo
root) and links the shared library next to this file.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libglq_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["api.cpp", "e8_codebook.cpp", "pack.cpp", "rht.hip", "dequant.hip", "gemv.hip", "gemv_lds.hip",
           "fused_decode.hip", "gemm.hip", "gemm_lds.hip", "gemm_shared.hip", "kv_attention.hip", "noalloc.hip", "gemv_mfma.hip"]

COMMON = ["-O3", "-fPIC", "-std=c++17", "-I" + INCLUDE, "-I" + CSRC, "-Wall", "-Wno-unused-function"]
# packed fp32 arithmetic stays off for all device code
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def _compile(src, verbose):
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON + (DEVICE if src.endswith(".hip") else []) + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    if verbose and r.stderr.strip():
        sys.stderr.write(r.stderr)
    return out


def build(verbose=False, jobs=8):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
