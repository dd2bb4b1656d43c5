import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def oracle_codebook():
    from oracle import e8
    return e8.codebook()


@pytest.fixture(scope="session")
def gpu_codebooks():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import e8_lattice_codebook_amd as glq
    return glq.Codebooks("cuda:0")


def pytest_sessionfinish(session, exitstatus):
    # with the debug library (GLQ_LIB_VARIANT=debug), every GPU test run in this process
    # also checks the device-side bounds checks: any failed check fails the session
    if os.environ.get("GLQ_LIB_VARIANT") != "debug":
        return
    from e8_lattice_codebook_amd import _lib
    if _lib._lib is None:
        return
    v = int(_lib.load().glq_debug_violations())
    print("\nglq_debug_violations: %d" % v)
    if v != 0:
        session.exitstatus = 1
