"""The debug build's device-side bounds checks (libglq_mi355x_debug.so, GLQ_DEBUG): one
call of each path, both index formats, with the oracle's check, and no failed check
(glq_debug_violations() == 0).  The debug library runs in a subprocess
(tests/gpu_debug_worker.py) so that it does not replace the release library this
process has loaded."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "e8_lattice_codebook_amd", "libglq_mi355x_debug.so")


def test_debug_build_bounds_checks():
    if not os.path.exists(LIB):
        pytest.skip("libglq_mi355x_debug.so is not built (e8_lattice_codebook_amd/build.py --variant debug)")
    env = dict(os.environ, GLQ_LIB_VARIANT="debug")
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "gpu_debug_worker.py")], env=env,
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    print(r.stdout[-4000:])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "violations 0" in r.stdout
