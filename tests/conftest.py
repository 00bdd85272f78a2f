import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(autouse=True)
def _device_status_clear(request):
    """GPU tests: the library's device status word (bits raised by a kernel
    that gave up a bounded wait) is cleared before the test and must still be
    clear after it."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    try:
        import torch
        if not torch.cuda.is_available():
            raise ImportError
        import bit_quantized_moe_diffrouter_amd as q
        q.lib()
    except Exception:
        yield
        return
    q.device_status(reset=True)
    yield
    assert q.device_status(reset=True) == 0, "a kernel raised the device status word"
