import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) GPU; runs the HIP library")


@pytest.fixture(scope="session")
def fp4():
    """The product binding, with libfp4.so built if (and only if) absent."""
    import block_scaled_fp4_amax_amd as F
    if not F.LIB_PATH.exists():
        from block_scaled_fp4_amax_amd import build
        build.build()
    F.lib()
    return F


@pytest.fixture(scope="session")
def oracle():
    from oracle import oracle as O
    O.lib()
    return O
