import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def gns_mod():
    """The HIP library binding; a GPU run must load the native library (no fallback)."""
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import muon_gram_ns_amd as g
    return g
