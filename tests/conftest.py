import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # A GPU test on a machine without a GPU fails loudly instead of skipping, so a
    # GPU run can never pass by not running the kernels.
    pass


@pytest.fixture(scope="session")
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test needs a visible ROCm GPU (torch.cuda.is_available() is False)")
    return torch.device("cuda:0")


def read_golden(name):
    """Parse a ``key: values`` fixture; repeated keys collect into lists of rows."""
    data = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            toks = val.split()
            data.setdefault(key.strip(), []).append(toks)
    return data
