import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def gpu():
    """GPU tests fail (not skip) when no GPU is visible: they are only
    selected with -m gpu, on a machine that has one."""
    import torch
    assert torch.cuda.is_available(), "GPU test selected on a machine without a visible GPU"
    import gemv_router_softmax_amd as moe
    moe.lib()   # the HIP library must be built and loadable
    return torch.device("cuda")
