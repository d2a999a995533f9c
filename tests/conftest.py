import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session", autouse=True)
def _host_libs():
    """Build the host-side helper libraries (synthetic inputs, CPU oracle) when
    they are missing; they compile in about a second."""
    import synth
    import synth.build
    import oracle
    import oracle.build
    if not os.path.exists(os.path.join(ROOT, "synth", "libmoe_synth.so")):
        synth.build.build()
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build.build()
    yield


@pytest.fixture(autouse=True)
def _guard_bands():
    """After a GPU test, check the guard bands around the buffers it
    allocated through gpu_util (a kernel writing past a buffer fails it)."""
    yield
    gu = sys.modules.get("gpu_util")
    if gu is not None:
        gu.check_guards()
