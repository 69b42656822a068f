import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (not skip) when run with -m gpu on a machine without a GPU;
    # without -m gpu they are deselected by the default expression in pytest.ini.
    pass


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; errors out if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import nvfp4_w4a4_moe_amd as nv4
    nv4.load()
    return nv4
