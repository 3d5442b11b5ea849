import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on a GPU: built in-tree before the run, loaded here.

    On a machine with a GPU a missing library is an error, not a skip.
    """
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from spatiotemporal_attention_vx_amd import binding
    return binding.load()
