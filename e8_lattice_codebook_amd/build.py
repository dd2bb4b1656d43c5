"""Build the gfx950 HIP library libglq_mi355x.so in-tree with hipcc.

Every call compiles every source again (object files go to _build/<variant>/ at the
repo root) and links the shared library next to this file.  Variants:
  release  libglq_mi355x.so        -O3
  debug    libglq_mi355x_debug.so  -O1 -DGLQ_DEBUG: device-side bounds checks count
                                   violations (glq_debug_violations) instead of trapping
  asan     libglq_mi355x_asan.so   the debug build with AddressSanitizer (and -g) on the
                                   host code only (device code is not instrumented); load
                                   it with the clang ASan runtime preloaded
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
# variant -> (library file, compile flags, link flags)
VARIANTS = {
    "release": (LIB_NAME, ["-O3"], []),
    "debug": ("libglq_mi355x_debug.so", ["-O1", "-DGLQ_DEBUG"], []),
    "asan": ("libglq_mi355x_asan.so",
             ["-O1", "-DGLQ_DEBUG", "-Xarch_host", "-g"]
             + "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split(),
             "-Xarch_host -fsanitize=address".split()),
}

SOURCES = ["api.cpp", "e8_codebook.cpp", "pack.cpp", "rht.hip", "dequant.hip", "gemv.hip", "gemv_lds.hip",
           "fused_decode.hip", "gemm.hip", "gemm_lds.hip", "gemm_shared.hip", "kv_attention.hip", "noalloc.hip", "gemv_i8.hip"]

COMMON = ["-fPIC", "-std=c++17", "-I" + INCLUDE, "-I" + CSRC, "-Wall", "-Wno-unused-function"]
# packed fp32 arithmetic stays off for all device code
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def lib_path(variant="release"):
    return os.path.join(PKG, VARIANTS[variant][0])


def _compile(src, verbose, variant):
    out = os.path.join(BUILD, variant, os.path.splitext(src)[0] + ".o")
    cmd = ([hipcc()] + VARIANTS[variant][1] + COMMON + (DEVICE if src.endswith(".hip") else [])
           + ["-c", os.path.join(CSRC, src), "-o", out])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    if verbose and r.stderr.strip():
        sys.stderr.write(r.stderr)
    return out


def build(verbose=False, jobs=8, variant="release"):
    os.makedirs(os.path.join(BUILD, variant), exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, variant), SOURCES))
    out = lib_path(variant)
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH] + VARIANTS[variant][2] + ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, out)
    return out


def build_all(verbose=False, jobs=8):
    """The release library, then the debug and host-ASan builds."""
    return [build(verbose, jobs, v) for v in ("release", "debug", "asan")]


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build the gfx950 library in-tree")
    ap.add_argument("--variant", choices=sorted(VARIANTS), default="release")
    ap.add_argument("--all", action="store_true", help="build every variant")
    a = ap.parse_args()
    print(build_all(verbose=True) if a.all else build(verbose=True, variant=a.variant))
