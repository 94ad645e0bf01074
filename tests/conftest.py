import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # The CPU helper libraries are built on demand (gcc) when they are missing.
    import gen
    import oracle
    if not os.path.exists(gen._LIB_PATH):
        gen.build()
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.get()


@pytest.fixture(scope="session")
def device():
    """cuda:0 with the HIP library loaded; GPU tests are skipped only on a host with no GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")
    import row_normalization_norm_amd as rn
    rn.lib()  # raises when librownorm.so is missing: never fall back
    return torch.device("cuda:0")


def pytest_sessionfinish(session, exitstatus):
    """With PARITY_REPORT=path, write every compared output's worst error as a fraction
    of its bound (one JSON object per line)."""
    path = os.environ.get("PARITY_REPORT")
    if not path or "parity" not in sys.modules:
        return
    import json
    from parity import REPORT
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        for r in REPORT:
            f.write(json.dumps(r) + "\n")
