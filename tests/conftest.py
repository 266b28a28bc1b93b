import shutil
import subprocess
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


@pytest.fixture(scope="session")
def rocrand_philox(tmp_path_factory):
    """run(seed, subsequence, count) -> uint32 [count, 4]: Philox4x32-10
    outputs of rocRAND's engine (built here from tests/philox_rocrand_ref.cpp),
    output n from counter (n, 0, subsequence_lo, subsequence_hi) under key
    seed. An implementation independent of the oracle."""
    import numpy as np
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(hipcc).exists():
        pytest.skip("hipcc not available to build the rocRAND reference")
    exe = tmp_path_factory.mktemp("philox") / "philox_ref"
    subprocess.run([hipcc, "-O1", str(ROOT / "tests" / "philox_rocrand_ref.cpp"), "-o", str(exe)], check=True,
                   capture_output=True)

    def run(seed, sub, count):
        out = subprocess.run([str(exe), str(seed), str(sub), str(count)], check=True, capture_output=True, text=True)
        return np.array([[int(w, 16) for w in line.split()] for line in out.stdout.splitlines()], np.uint32)
    return run
