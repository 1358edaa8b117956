import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _device_status_clean(request):
    """Every GPU test starts with the library's device-side status bits clear
    and must end with none raised (a bounded wait that gave up, or a state
    index outside the pool); a test that raises them on purpose clears them."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import linear_attention_state_amd as gdn

    gdn.gdn_device_status(clear=True)
    yield
    bits = gdn.gdn_device_status(clear=True)
    assert bits == 0, "device status bits 0x%x were raised during the test" % bits
