import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library")
    config.addinivalue_line("markers", "slow: CPU-heavy oracle work (tens of seconds)")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (not skip) when run with -m gpu on a machine without
    # a GPU: a silent skip would hide a missing native path.
    pass


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library binding, on a machine that has the GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch.cuda.is_available() is False")
    import io_aware_exact_fwd_amd as attn
    rc = attn.device_check(torch.cuda.current_device())
    assert rc == 0, attn.strerror(rc)
    return attn
