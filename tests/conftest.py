import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size CPU work (tens of seconds)")


@pytest.fixture(scope="session", autouse=True)
def _built_host_libs():
    """The CPU-side libraries (generator, oracle) are plain C; build them if absent."""
    import oracle
    from mxfp4_routed_expert_sqrt_amd import synth
    if not os.path.exists(oracle._LIB):
        oracle.build()
    if not os.path.exists(synth._LIB_PATH):
        from mxfp4_routed_expert_sqrt_amd import build as pkg_build
        pkg_build.build_synth()
    yield
