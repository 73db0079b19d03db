import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line(
        "markers", "slow: long CPU run (still part of the default CPU suite)")


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.build(force=False)
    return oracle.default()


@pytest.fixture(scope="session")
def pins_exe(tmp_path_factory):
    """The exhaustive pin checker, compiled for this session."""
    d = tmp_path_factory.mktemp("pins")
    exe = str(d / "exhaustive_pins")
    src = os.path.join(ROOT, "tests", "pins", "exhaustive_pins.c")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe, src,
                    "-lm", "-ldl"], check=True)
    return exe
