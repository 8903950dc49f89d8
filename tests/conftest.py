import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_runtest_setup(item):
    # GPU tests fail loudly (never skip) when no device is visible.
    if item.get_closest_marker("gpu") is not None:
        import torch
        if not torch.cuda.is_available():
            import pytest
            pytest.fail("GPU test but torch.cuda.is_available() is False")
