import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # A gpu-marked test on a machine without a GPU fails loudly instead of silently passing; the
    # CPU suite is run with -m "not gpu", which deselects them before this point.
    pass


@pytest.fixture(scope="session")
def lib():
    """The HIP library binding; a GPU test that cannot load it fails (no fallback)."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but no GPU is visible")
    import nf4_dequant_gemm_amd as m
    return m
