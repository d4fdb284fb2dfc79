import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def pages():
    with open(os.path.join(ROOT, "tests", "golden", "pages_figures.json")) as f:
        return json.load(f)


def _ensure_built():
    lib = os.path.join(ROOT, "entropy_coding_amd", "libkvc.so")
    if not os.path.exists(lib):
        from entropy_coding_amd import build
        build.build()
    return lib


@pytest.fixture(scope="session")
def kvc():
    """The binding over the built library (built first if missing)."""
    _ensure_built()
    from entropy_coding_amd import kvc as k
    return k


@pytest.fixture(scope="session")
def cuda(kvc):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")
