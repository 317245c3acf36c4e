import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _ensure_built():
    # Load what is built; build only if nothing is (the build step normally runs first).
    from block_scaled_fp4_gemv_amd import _build
    if not os.path.exists(_build.SYNTH_LIB):
        _build.build_synth()
    if _build.hip_sources() and not os.path.exists(_build.MOE_LIB):
        _build.build_moe()


_ensure_built()


@pytest.fixture(scope="session")
def synth():
    from block_scaled_fp4_gemv_amd import synth as s
    return s
